// Ragged MLA prefill attention, fp32 inputs, for gfx950.
//
// Same definition as the bf16 kernel (ragged prefill with LSE,
// "vllm.v1.attention.backends.mla.prefill.flashinfer", run() with
// return_lse; head dims 192 / 128 from sglang issue 3849) computed entirely
// in fp32, so fp32 inputs are never rounded to bf16. It serves accuracy
// (fp32 callers, the 1e-4 / 1e-5 bounds); the bf16 kernel is the throughput
// path.
//
// Design (MI355X):
//  * Both products run on the fp32 matrix cores, v_mfma_f32_32x32x2f32
//    (fp32 operands, fp32 accumulation). One workgroup = 4 waves x 32 query
//    rows (128-row tiles), its heads one after the other.
//  * Scores are computed transposed, S^T = K Q^T, 96 k-steps of 2 dims:
//    A = K (32 keys x 2 dims, from LDS), B = Q (2 dims x 32 queries, 96
//    VGPRs per lane). The two dims of a k-step are d and d + 4 of each
//    8-dim block, so every lane reads its K values as one 16-byte LDS load
//    per 4 k-steps and holds the matching Q values.
//  * The S^T accumulator, slot (i, half g) = key 8 (i/4) + 4 g + i%4 of the
//    lane's query column, is exponentiated in place and is directly the B
//    operand of O^T = V^T P^T (16 k-steps of 2 keys): k-step t pairs the
//    keys held in slot t of the two lane halves, and the A operand reads
//    those two V rows from LDS, one fp32 value per lane.
//  * K and V tiles of 32 keys are staged in LDS by the whole workgroup with
//    16-byte loads (rows padded to 196 and 136 floats, so the fragment reads
//    are free of bank conflicts); keys past the sequence end are zero.
//  * Online softmax in base 2 with sm_scale * log2(e) folded in, the O and
//    row-sum rescale on every tile where the maximum moves (exact fp32;
//    the row sums of the two lane halves are combined at the end).
//  * Waves skip the arithmetic of tiles beyond their last visible key (they
//    still take part in the loads and barriers); rows with no visible key
//    get O = 0 and LSE = -inf.
#include "internal.h"

namespace mla {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;        // 32 query rows per wave
constexpr int kBN = 32;                 // keys per tile
constexpr int kKStride = kDqk + 4;      // 196 floats: 784-byte rows
constexpr int kVStride = kDvo + 8;      // 136 floats: rows 4 apart differ by 128 B mod 256
constexpr int kQRegs = kDqk / 2;        // 96 Q values per lane
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int lim_of(int r, int diag0, int kv_len) {
    int n = diag0 + r + 1;
    n = n < 0 ? 0 : n;
    return n > kv_len ? kv_len : n;
}

template <bool kPaged>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp32_kernel(const WorkItem* __restrict__ items, const float* __restrict__ q,
                         const float* __restrict__ k, const float* __restrict__ v,
                         float* __restrict__ out, float* __restrict__ lse, int num_heads,
                         float scale_log2, PagedKv pg) {
    __shared__ __attribute__((aligned(16))) float ks[kBN * kKStride];
    __shared__ __attribute__((aligned(16))) float vs[kBN * kVStride];

    const WorkItem it = items[blockIdx.x];
    if (it.n_rows <= 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int H = num_heads;
    const int row_w0 = wave * 32;
    int wave_rows = it.n_rows - row_w0;
    wave_rows = wave_rows < 0 ? 0 : (wave_rows > 32 ? 32 : wave_rows);
    // keys the wave's last row sees: tiles at or past it are skipped
    const int wave_hi = wave_rows > 0 ? lim_of(row_w0 + wave_rows - 1, it.diag0, it.kv_len) : 0;
    const int my_row = row_w0 + l32;
    const int my_lim = lim_of(my_row, it.diag0, it.kv_len);
    // rows past the tile's end read its last row (never stored)
    const int q_row = it.q_row0 + (my_row < it.n_rows ? my_row : it.n_rows - 1);

    // K/V row (token index in the cache, head 0) of key `key` (< kv_len)
    auto kv_row = [&](int key) -> int64_t {
        if constexpr (kPaged) {
            int pgi = pg.block_table[(int64_t)it.kv_start * pg.max_pages + key / pg.page_size];
            pgi = pgi < 0 ? 0 : (pgi >= pg.num_pages ? pg.num_pages - 1 : pgi);
            return ((int64_t)pgi * pg.page_size + key % pg.page_size) * H;
        } else {
            return ((int64_t)it.kv_start + key) * H;
        }
    };

    for (int head = it.head0; head < it.head0 + it.n_heads; ++head) {
        // Q values of k-step (u, e): dim 8u + 4g + e of this lane's query row
        float qf[kQRegs];
        {
            const float* src = q + ((int64_t)q_row * H + head) * kDqk + 4 * g;
#pragma unroll
            for (int u = 0; u < kDqk / 8; ++u) {
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 8 * u);
                qf[4 * u + 0] = x[0];
                qf[4 * u + 1] = x[1];
                qf[4 * u + 2] = x[2];
                qf[4 * u + 3] = x[3];
            }
        }
        f32x16_t oacc[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
        float m_run = -INFINITY, l_run = 0.f;

        for (int key0 = 0; key0 < it.kv_hi; key0 += kBN) {
            __syncthreads();   // the previous tile's reads are done
            // K tile: 32 rows x 48 float4; V tile: 32 rows x 32 float4
            for (int u = tid; u < kBN * (kDqk / 4); u += kThreads) {
                const int r = u / (kDqk / 4), c = u % (kDqk / 4);
                const int key = key0 + r;
                *reinterpret_cast<f32x4_t*>(&ks[r * kKStride + 4 * c]) =
                    key < it.kv_len ? *reinterpret_cast<const f32x4_t*>(k + (kv_row(key) + head) * kDqk + 4 * c)
                                    : f32x4_t{};
            }
            for (int u = tid; u < kBN * (kDvo / 4); u += kThreads) {
                const int r = u / (kDvo / 4), c = u % (kDvo / 4);
                const int key = key0 + r;
                *reinterpret_cast<f32x4_t*>(&vs[r * kVStride + 4 * c]) =
                    key < it.kv_len ? *reinterpret_cast<const f32x4_t*>(v + (kv_row(key) + head) * kDvo + 4 * c)
                                    : f32x4_t{};
            }
            __syncthreads();
            if (key0 >= wave_hi) continue;   // wave-uniform: no row of this wave sees the tile

            // S^T = K Q^T: lane (key l32, half g) supplies K[key][8u + 4g + e]
            f32x16_t sacc = f32x16_t{};
            const float* krow = &ks[l32 * kKStride + 4 * g];
#pragma unroll
            for (int u = 0; u < kDqk / 8; ++u) {
                const f32x4_t a = *reinterpret_cast<const f32x4_t*>(krow + 8 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[4 * u + e], sacc, 0, 0, 0);
            }
            // mask: slot i holds key key0 + 8 (i/4) + 4 g + i%4 of query row my_row
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + (i >> 2) * 8 + g * 4 + (i & 3);
                sacc[i] = key < my_lim ? sacc[i] * scale_log2 : -INFINITY;
                mt = fmaxf(mt, sacc[i]);
            }
            mt = xor32_max(mt);
            const float m_new = fmaxf(m_run, mt);
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            if (m_new != m_run) {
                const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
                m_run = m_new;
            }
            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sacc[i] = __builtin_amdgcn_exp2f(sacc[i] - msub);
                lsum += sacc[i];
            }
            l_run += lsum;
            // O^T = V^T P^T: k-step t pairs the keys of slot t in the two
            // halves; lane (dim l32, half g) reads V[key(t, g)][32 db + l32]
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const float* vrow = &vs[((t >> 2) * 8 + g * 4 + (t & 3)) * kVStride + l32];
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db], sacc[t], oacc[db], 0, 0, 0);
            }
        }

        // epilogue: O = acc / l, LSE = (m + log2 l) ln 2; the accumulator
        // slot (i, g) of dv block db is dim 32 db + 8 (i/4) + 4 g + i%4
        if (wave_rows > 0) {
            const float ltot = xor32_sum(l_run);
            if (my_row < it.n_rows) {
                const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
                const int64_t orow = (int64_t)(it.q_row0 + my_row) * H + head;
                float* dst = out + orow * kDvo;
#pragma unroll
                for (int db = 0; db < 4; ++db) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const f32x4_t o4 = {oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                                            oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv};
                        *reinterpret_cast<f32x4_t*>(dst + 32 * db + 8 * a + 4 * g) = o4;
                    }
                }
                if (g == 0 && lse != nullptr)
                    lse[orow] = ltot > 0.f ? (m_run + __log2f(ltot)) * kLn2 : -INFINITY;
            }
        }
    }
}

}  // namespace

int prefill_fp32_block_m() { return kBM; }

hipError_t launch_prefill_fp32(const WorkItem* items, int64_t n_items, const void* q,
                               const void* k, const void* v, void* out, float* lse,
                               int num_heads, float sm_scale, hipStream_t stream,
                               const PagedKv* paged) {
    if (n_items <= 0) return hipSuccess;
    if (n_items > 0x7fffffff) return hipErrorInvalidValue;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    const PagedKv pg = paged != nullptr ? *paged : PagedKv{nullptr, 0, 0, 0};
    if (paged != nullptr)
        hipLaunchKernelGGL(prefill_fp32_kernel<true>, dim3((unsigned)n_items), dim3(kThreads), 0,
                           stream, items, static_cast<const float*>(q),
                           static_cast<const float*>(k), static_cast<const float*>(v),
                           static_cast<float*>(out), lse, num_heads, scale_log2, pg);
    else
        hipLaunchKernelGGL(prefill_fp32_kernel<false>, dim3((unsigned)n_items), dim3(kThreads), 0,
                           stream, items, static_cast<const float*>(q),
                           static_cast<const float*>(k), static_cast<const float*>(v),
                           static_cast<float*>(out), lse, num_heads, scale_log2, pg);
    return hipGetLastError();
}

}  // namespace mla
