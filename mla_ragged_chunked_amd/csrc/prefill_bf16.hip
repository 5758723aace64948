// Ragged MLA prefill attention, bf16 inputs, for gfx950 (CDNA4).
//
// Computes, per work item (one query tile of one (sequence, head)), flash-
// style attention with Dqk = 192 and Dvo = 128: S = sm_scale * Q K^T over the
// visible keys (bottom-right causal or all), online softmax in fp32, O = P V,
// and the natural-log LSE per row. This is the ragged prefill of
// "vllm.v1.attention.backends.mla.prefill.flashinfer" (run() with
// return_lse) at the MLA head dims of "[DeepseekR1] How ragged prefill
// manage kv_cache?" (192 for query/key, 128 for value/output).
//
// Design (MI355X):
//  * One workgroup = 4 waves x 64 query rows. Each wave keeps its 64 Q rows
//    in VGPRs as MFMA B operands for the whole item (96 VGPRs).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//    32 queries. In the accumulator each lane then owns one query column and
//    16 keys, so row max / row sum are in-lane plus one exchange between the
//    two 32-lane halves.
//  * The same accumulator, rounded to bf16, is directly the B operand of
//    O^T = V^T P^T, provided V^T's key columns in LDS are permuted to match
//    the accumulator's row order: accumulator slot (i, half g) of a 32-key
//    block holds key 8*(i/4) + 4*g + (i%4); the PV k-slot 8*g + e of MFMA m
//    must hold key 16*m + 8*(e/4) + 4*g + (e%4). Storing key j at LDS column
//    sigma(j) = j with bits 2 and 3 swapped makes every A fragment one
//    contiguous 16-byte read.
//  * K (row-major, 400-byte pitch) and V^T (key-permuted, 80-byte pitch)
//    tiles of 32 keys are staged in LDS with two stages: tile t+1 is fetched
//    into VGPRs while tile t is computed, then written to the other stage;
//    one barrier per tile. Pitches are padded so fragment reads of
//    consecutive rows fall in distinct banks.
//  * Online softmax in base 2 with sm_scale * log2(e) folded into one FMA;
//    the running max is only raised when it grows by more than 2^8 (the
//    stale max keeps every p <= 256, exact after the final division), so the
//    O rescale is skipped on most tiles. The row sum is accumulated from the
//    bf16-rounded p that enter the MFMA, so O is normalised by exactly the
//    weights it was built from.
//  * Keys past the sequence end are zero-filled (no NaN can reach the PV
//    product); rows with no visible key get O = 0, LSE = -inf.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 64;
constexpr int kBM = kWaves * kRowsPerWave;
static_assert(kBM == kBf16BlockM, "tile height must match the planner");
constexpr int kBN = 32;                             // keys per KV tile
constexpr int kKSteps = kDqk / 16;                  // 12 MFMA k-steps over 192 dims
constexpr int kKPitch = kDqk * 2 + 16;              // bytes per K row in LDS
constexpr int kVPitch = kBN * 2 + 16;               // bytes per V^T row in LDS
constexpr int kKBytes = kBN * kKPitch;
constexpr int kVBytes = kDvo * kVPitch;
constexpr int kStage = kKBytes + kVBytes;
constexpr int kKChunks = kBN * (kDqk / 8);          // 16-byte chunks per K tile
constexpr int kKPerThread = kKChunks / kThreads;
constexpr int kVUnits = (kBN / 2) * (kDvo / 8);     // (key pair, 16-byte chunk) units
constexpr int kVPerThread = kVUnits / kThreads;
static_assert(kKChunks % kThreads == 0 && kVUnits % kThreads == 0, "staging split");
constexpr float kLazyRescale = 8.0f;                // log2 units
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int sigma(int j) {
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ int lim_of(int r, int diag0, int kv_len) {
    int n = diag0 + r + 1;
    n = n < 0 ? 0 : n;
    return n > kv_len ? kv_len : n;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_bf16_kernel(const WorkItem* __restrict__ items, const uint16_t* __restrict__ q,
                         const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                         uint16_t* __restrict__ out, float* __restrict__ lse, int num_heads,
                         float scale_log2) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

    const WorkItem it = items[blockIdx.x];
    if (it.n_rows <= 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int H = num_heads;
    const int row_w0 = wave * kRowsPerWave;
    int wave_rows = it.n_rows - row_w0;
    wave_rows = wave_rows < 0 ? 0 : (wave_rows > kRowsPerWave ? kRowsPerWave : wave_rows);
    const bool wave_active = wave_rows > 0;
    const int wave_lo = wave_active ? lim_of(row_w0, it.diag0, it.kv_len) : 0;
    const int wave_hi = wave_active ? lim_of(row_w0 + wave_rows - 1, it.diag0, it.kv_len) : 0;

    // ---- Q fragments: rows row_w0 + 32*qb + l32, dims 16*s + 8*g .. +8
    bf16x8_t qf[2][kKSteps];
    int my_lim[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int r = row_w0 + qb * 32 + l32;
        my_lim[qb] = lim_of(r, it.diag0, it.kv_len);
        if (r < it.n_rows) {
            const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(
                q + ((int64_t)(it.q_row0 + r) * H + it.head) * kDqk);
#pragma unroll
            for (int s = 0; s < kKSteps; ++s) qf[qb][s] = src[s * 2 + g];
        } else {
#pragma unroll
            for (int s = 0; s < kKSteps; ++s) qf[qb][s] = bf16x8_t{};
        }
    }

    f32x16_t oacc[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x16_t{};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    // ---- K/V staging through VGPRs
    u32x4_t kreg[kKPerThread];
    u32x4_t vreg[kVPerThread][2];
    const int64_t kv_row_base = (int64_t)it.kv_start * H + it.head;

    auto load_tile = [&](int key0) {
#pragma unroll
        for (int j = 0; j < kKPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int row = u / (kDqk / 8);
            const int c = u % (kDqk / 8);
            const int key = key0 + row;
            if (key < it.kv_len) {
                kreg[j] = *reinterpret_cast<const u32x4_t*>(
                    k + (kv_row_base + (int64_t)key * H) * kDqk + c * 8);
            } else {
                kreg[j] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < kVPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int p = u % (kBN / 2);
            const int c = u / (kBN / 2);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int key = key0 + 2 * p + h2;
                if (key < it.kv_len) {
                    vreg[j][h2] = *reinterpret_cast<const u32x4_t*>(
                        v + (kv_row_base + (int64_t)key * H) * kDvo + c * 8);
                } else {
                    vreg[j][h2] = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
    };

    auto store_tile = [&](int stage) {
        uint8_t* ks = smem + stage * kStage;
        uint8_t* vs = ks + kKBytes;
#pragma unroll
        for (int j = 0; j < kKPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int row = u / (kDqk / 8);
            const int c = u % (kDqk / 8);
            *reinterpret_cast<u32x4_t*>(ks + row * kKPitch + c * 16) = kreg[j];
        }
#pragma unroll
        for (int j = 0; j < kVPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int p = u % (kBN / 2);
            const int c = u / (kBN / 2);
            const int col = sigma(2 * p);    // sigma(2p + 1) == sigma(2p) + 1
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w0 = vreg[j][0][e >> 1];
                const uint32_t w1 = vreg[j][1][e >> 1];
                const uint32_t packed = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                                : ((w0 & 0xffffu) | (w1 << 16));
                *reinterpret_cast<uint32_t*>(vs + (c * 8 + e) * kVPitch + col * 2) = packed;
            }
        }
    };

    const int n_tiles = (it.kv_hi + kBN - 1) / kBN;
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = 0; kt < n_tiles; ++kt) {
        const int key0 = kt * kBN;
        const bool has_next = kt + 1 < n_tiles;
        if (has_next) load_tile(key0 + kBN);

        if (wave_active && key0 < wave_hi) {
            const uint8_t* ks = smem + (kt & 1) * kStage;
            const uint8_t* vs = ks + kKBytes;

            // S^T = K Q^T for 32 keys x 64 queries
            f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
            for (int s = 0; s < kKSteps; ++s) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                    ks + l32 * kKPitch + (s * 16 + g * 8) * 2);
                sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][s], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][s], sacc[1], 0, 0, 0);
            }

            const bool need_mask = key0 + kBN > wave_lo;
            bf16x8_t pf[2][2];
            bool any_rescale = false;
            float alpha[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                if (need_mask) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + (i >> 2) * 8 + g * 4 + (i & 3);
                        if (key >= my_lim[qb]) sacc[qb][i] = -INFINITY;
                    }
                }
                float mx = sacc[qb][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[qb][i]);
                mx = fmaxf(mx, xor32(mx));
                const float m_tile = mx * scale_log2;    // -inf stays -inf (scale > 0)
                const float m_old = m_run[qb];
                const bool raise = m_tile > m_old + kLazyRescale;
                const float m_new = raise ? m_tile : m_old;
                alpha[qb] = raise ? __builtin_amdgcn_exp2f(m_old - m_new) : 1.0f;
                any_rescale |= raise;
                m_run[qb] = m_new;
                const float msub = m_new == -INFINITY ? 0.0f : m_new;

                float lsum = 0.f;
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    bf16x8_t frag;
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(sacc[qb][mm * 8 + e], scale_log2, -msub));
                        const float p1 = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(sacc[qb][mm * 8 + e + 1], scale_log2, -msub));
                        const bf16x2_t pk = {(__bf16)p0, (__bf16)p1};
                        frag[e] = pk[0];
                        frag[e + 1] = pk[1];
                        lsum += (float)pk[0] + (float)pk[1];
                    }
                    pf[qb][mm] = frag;
                }
                l_run[qb] = l_run[qb] * alpha[qb] + lsum;
            }

            // wave-uniform: rescale O only when some row raised its max
            if (__any(any_rescale)) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] *= alpha[qb];
            }

            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < 4; ++db) {
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                        vs + (db * 32 + l32) * kVPitch + (mm * 16 + g * 8) * 2);
                    oacc[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[0][mm], oacc[db][0], 0, 0, 0);
                    oacc[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[1][mm], oacc[db][1], 0, 0, 0);
                }
            }
        }

        if (has_next) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
    if (!wave_active) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int r = row_w0 + qb * 32 + l32;
        const float ltot = l_run[qb] + xor32(l_run[qb]);
        if (r >= it.n_rows) continue;
        const float inv = ltot > 0.f ? 1.0f / ltot : 0.0f;
        const int64_t orow = (int64_t)(it.q_row0 + r) * H + it.head;
        uint16_t* dst = out + orow * kDvo;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int dv = db * 32 + grp * 8 + g * 4;
                bf16x4_t o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][qb][grp * 4 + e] * inv);
                *reinterpret_cast<bf16x4_t*>(dst + dv) = o4;
            }
        }
        if (g == 0 && lse != nullptr)
            lse[orow] = ltot > 0.f ? (m_run[qb] + __log2f(ltot)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const WorkItem* items, int64_t n_items, const void* q,
                               const void* k, const void* v, void* out, float* lse,
                               int num_heads, float sm_scale, hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    if (n_items > 0x7fffffff) return hipErrorInvalidValue;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)n_items), dim3(kThreads), 0, stream,
                       items, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse,
                       num_heads, scale_log2);
    return hipGetLastError();
}

}  // namespace mla
