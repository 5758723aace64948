// MLA KV decompression for gfx950: per-head K_nope and V from the latent cache.
//
// The cache holds a 512-dim compressed latent per token plus 64 RoPE key
// dims, while ragged prefill runs MHA with 192-dim keys and 128-dim values
// ("[DeepseekR1] How ragged prefill manage kv_cache?", sglang issue 3849:
// the question whether the latent is decompressed for every chunked-prefill
// pass). This kernel performs that decompression:
//   K[t,h,0:128]   = c_kv[t,:] . W_UK[:, h*128 : h*128+128]
//   K[t,h,128:192] = k_rope[t,:]               (one copy per head)
//   V[t,h,:]       = c_kv[t,:] . W_UV[:, h*128 : h*128+128]
// as two bf16 MFMA GEMMs ([T,512] x [512, H*128]) with fp32 accumulation.
//
// Tiling: one workgroup = one head x 256 tokens of either K or V (grid.z).
// The product is computed transposed, C^T[n][t] = sum_c W[c][n] c_kv[t][c],
// with v_mfma_f32_32x32x16_bf16: A = W^T (n rows, latent dims along k), B =
// c_kv^T (token columns, latent dims along k). c_kv rows are k-contiguous
// already; W is n-contiguous, so each 32-dim slice of W is transposed into
// LDS while staging. Each accumulator lane then owns one token and groups of
// four consecutive output dims, written as 8-byte stores. Four waves split
// the 128 x 256 tile 2 x 2 (64 dims x 128 tokens each).
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTT = 256;                    // tokens per tile
constexpr int kNT = 128;                    // output dims per tile (one head)
constexpr int kKC = 32;                     // latent dims per stage
constexpr int kWPitch = kKC * 2 + 16;       // bytes per W^T row in LDS
constexpr int kCPitch = kKC * 2 + 16;       // bytes per c_kv row in LDS
constexpr int kWBytes = kNT * kWPitch;
constexpr int kCBytes = kTT * kCPitch;
constexpr int kStage = kWBytes + kCBytes;
constexpr int kWUnits = (kKC / 2) * (kNT / 8);        // (latent pair, 8-dim chunk)
constexpr int kWPerThread = kWUnits / kThreads;       // 1
constexpr int kCChunks = kTT * (kKC / 8);             // 16-byte chunks of c_kv
constexpr int kCPerThread = kCChunks / kThreads;      // 4
static_assert(kWUnits % kThreads == 0 && kCChunks % kThreads == 0, "staging split");

__global__ __launch_bounds__(kThreads) void decompress_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_rope,
    const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv, int num_tokens,
    int num_heads, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int t0 = blockIdx.x * kTT;
    const int head = blockIdx.y;
    const bool is_v = blockIdx.z == 1;
    const uint16_t* w = is_v ? w_uv : w_uk;
    const int H = num_heads;
    const int64_t wcols = (int64_t)H * kNT;
    const int wn = wave & 1;     // dims  [64*wn, +64)
    const int wt = wave >> 1;    // tokens [128*wt, +128)

    u32x4_t wreg[kWPerThread][2];
    u32x4_t creg[kCPerThread];

    auto load_stage = [&](int c0) {
#pragma unroll
        for (int j = 0; j < kWPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int p = u % (kKC / 2);
            const int nc = u / (kKC / 2);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                wreg[j][h2] = *reinterpret_cast<const u32x4_t*>(
                    w + (int64_t)(c0 + 2 * p + h2) * wcols + (int64_t)head * kNT + nc * 8);
        }
#pragma unroll
        for (int j = 0; j < kCPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int row = u / (kKC / 8);
            const int c = u % (kKC / 8);
            const int t = t0 + row;
            creg[j] = t < num_tokens
                          ? *reinterpret_cast<const u32x4_t*>(c_kv + (int64_t)t * kDlat + c0 + c * 8)
                          : u32x4_t{0u, 0u, 0u, 0u};
        }
    };

    auto store_stage = [&](int stage) {
        uint8_t* ws = smem + stage * kStage;
        uint8_t* cs = ws + kWBytes;
#pragma unroll
        for (int j = 0; j < kWPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int p = u % (kKC / 2);
            const int nc = u / (kKC / 2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w0 = wreg[j][0][e >> 1];
                const uint32_t w1 = wreg[j][1][e >> 1];
                const uint32_t packed = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                                : ((w0 & 0xffffu) | (w1 << 16));
                *reinterpret_cast<uint32_t*>(ws + (nc * 8 + e) * kWPitch + 2 * p * 2) = packed;
            }
        }
#pragma unroll
        for (int j = 0; j < kCPerThread; ++j) {
            const int u = tid + j * kThreads;
            const int row = u / (kKC / 8);
            const int c = u % (kKC / 8);
            *reinterpret_cast<u32x4_t*>(cs + row * kCPitch + c * 16) = creg[j];
        }
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x16_t{};

    constexpr int kStages = kDlat / kKC;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < kStages; ++st) {
        const bool has_next = st + 1 < kStages;
        if (has_next) load_stage((st + 1) * kKC);
        const uint8_t* ws = smem + (st & 1) * kStage;
        const uint8_t* cs = ws + kWBytes;
#pragma unroll
        for (int ks = 0; ks < kKC / 16; ++ks) {
            bf16x8_t a[2], b[4];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                a[nb] = *reinterpret_cast<const bf16x8_t*>(
                    ws + (wn * 64 + nb * 32 + l32) * kWPitch + (ks * 16 + g * 8) * 2);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                b[tb] = *reinterpret_cast<const bf16x8_t*>(
                    cs + (wt * 128 + tb * 32 + l32) * kCPitch + (ks * 16 + g * 8) * 2);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[nb], b[tb], acc[nb][tb], 0, 0, 0);
        }
        if (has_next) store_stage((st + 1) & 1);
        __syncthreads();
    }

    // epilogue: lane owns token t = tile col, dims in groups of 4
    const int out_dim = is_v ? kDvo : kDqk;
    uint16_t* dst_base = is_v ? v_out : k_out;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int t = t0 + wt * 128 + tb * 32 + l32;
        if (t >= num_tokens) continue;
        uint16_t* dst = dst_base + ((int64_t)t * H + head) * out_dim;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int n = wn * 64 + nb * 32 + grp * 8 + g * 4;
                bf16x4_t o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = (__bf16)acc[nb][tb][grp * 4 + e];
                *reinterpret_cast<bf16x4_t*>(dst + n) = o4;
            }
        }
    }

    // K workgroups also place k_rope after the NoPE part, for their tokens
    if (!is_v) {
        constexpr int kChunksPerTok = kDrope * 2 / 16;   // 8
        for (int u = tid; u < kTT * kChunksPerTok; u += kThreads) {
            const int row = u / kChunksPerTok;
            const int c = u % kChunksPerTok;
            const int t = t0 + row;
            if (t >= num_tokens) continue;
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(k_rope + (int64_t)t * kDrope + c * 8);
            *reinterpret_cast<u32x4_t*>(k_out + ((int64_t)t * H + head) * kDqk + kDnope + c * 8) = x;
        }
    }
}

}  // namespace

hipError_t launch_decompress(const void* c_kv, const void* k_rope, const void* w_uk,
                             const void* w_uv, int64_t num_tokens, int num_heads, void* k_out,
                             void* v_out, hipStream_t stream) {
    if (num_tokens <= 0) return hipSuccess;
    const int64_t tiles = (num_tokens + kTT - 1) / kTT;
    if (tiles > 0x7fffffff || num_heads > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decompress_kernel, dim3((unsigned)tiles, (unsigned)num_heads, 2),
                       dim3(kThreads), 0, stream, static_cast<const uint16_t*>(c_kv),
                       static_cast<const uint16_t*>(k_rope), static_cast<const uint16_t*>(w_uk),
                       static_cast<const uint16_t*>(w_uv), (int)num_tokens, num_heads,
                       static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
    return hipGetLastError();
}

}  // namespace mla
