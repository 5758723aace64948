// merge_state for gfx950: combine two attention states over disjoint key sets.
//
// Chunked prefill runs one causal pass over the new tokens and one
// non-causal pass per context chunk, each returning (O, LSE)
// ("vllm.v1.attention.backends.mla.prefill.flashinfer",
// run_prefill_context_chunk returns the pair for every chunk; sglang issue
// 3849 uses forward_return_lse for chunked prefill). The caller then folds
// the partial states with the log-sum-exp weighted combination:
//   lse = ln(e^a + e^b),  o = e^(a - lse) o_a + e^(b - lse) o_b,
// where a side with LSE = -inf carries weight 0 and both -inf give o = 0,
// lse = -inf.
//
// Pure HBM streaming: every row of 128 values is read twice and written once.
// Each lane moves one 16-byte chunk per operand (8 bf16 or 4 fp32) with
// non-temporal loads and stores (the data is touched once), and the grid
// covers every chunk of a batch of the bench's size at once (measured on
// MI355X: 6.5 TB/s, against 5.8 with two chunks per lane over half the grid
// and 5.4 with four over a quarter). The lanes of one row sit in one wave, so
// an in-place LSE write cannot overtake a read of the same row: every lane of
// the wave has loaded before any lane stores.
#include "internal.h"

namespace mla {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

template <bool kBf16>
__device__ __forceinline__ void merge_row_chunk(const u32x4_t xa, const u32x4_t xb, float a, float b,
                                                u32x4_t& res, float& out_lse) {
    const float mx = fmaxf(a, b);
    float wa = 0.f, wb = 0.f;
    out_lse = -INFINITY;
    if (mx != -INFINITY) {
        const float ea = __builtin_amdgcn_exp2f((a - mx) * kLog2e);   // exp(-inf) = 0
        const float eb = __builtin_amdgcn_exp2f((b - mx) * kLog2e);
        const float sum = ea + eb;
        const float inv = 1.0f / sum;
        wa = ea * inv;
        wb = eb * inv;
        out_lse = mx + __log2f(sum) * kLn2;
    }
    if constexpr (kBf16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float lo = 0.f, hi = 0.f;
            if (wa != 0.f) { lo += wa * bf16_lo(xa[w]); hi += wa * bf16_hi(xa[w]); }
            if (wb != 0.f) { lo += wb * bf16_lo(xb[w]); hi += wb * bf16_hi(xb[w]); }
            res[w] = pack_bf16(lo, hi);
        }
    } else {
        const f32x4_t fa = __builtin_bit_cast(f32x4_t, xa);
        const f32x4_t fb = __builtin_bit_cast(f32x4_t, xb);
        f32x4_t r;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float x = 0.f;
            if (wa != 0.f) x += wa * fa[w];
            if (wb != 0.f) x += wb * fb[w];
            r[w] = x;
        }
        res = __builtin_bit_cast(u32x4_t, r);
    }
}

// No pointer is declared __restrict__: o may alias o_a or o_b and lse may
// alias lse_a or lse_b (an in-place merge). Each output chunk depends only on
// the same row's inputs, loaded by the same lane (the LSE by every lane of
// the row's wave) before that lane stores.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
    float* lse, int64_t num_rows) {
    constexpr int kLanesPerRow = kBf16 ? kDvo * 2 / 16 : kDvo * 4 / 16;
    const int64_t total = num_rows * kLanesPerRow;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const u32x4_t* pa = reinterpret_cast<const u32x4_t*>(o_a);
    const u32x4_t* pb = reinterpret_cast<const u32x4_t*>(o_b);
    u32x4_t* po = reinterpret_cast<u32x4_t*>(o);
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += stride) {
        const int64_t row = idx / kLanesPerRow;
        const u32x4_t xa = __builtin_nontemporal_load(pa + idx);
        const u32x4_t xb = __builtin_nontemporal_load(pb + idx);
        u32x4_t res;
        float out_lse;
        merge_row_chunk<kBf16>(xa, xb, lse_a[row], lse_b[row], res, out_lse);
        __builtin_nontemporal_store(res, po + idx);
        if (idx % kLanesPerRow == 0) lse[row] = out_lse;
    }
}

}  // namespace

hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                        void* o, float* lse, int64_t num_rows, int dtype_bf16,
                        hipStream_t stream) {
    if (num_rows <= 0) return hipSuccess;
    const int64_t lanes_per_row = dtype_bf16 ? kDvo * 2 / 16 : kDvo * 4 / 16;
    const int64_t blocks_needed = (num_rows * lanes_per_row + kThreads - 1) / kThreads;
    // one chunk per lane in a single pass up to 2^20 workgroups (16M bf16
    // rows), looping beyond
    const int64_t max_blocks = int64_t(1) << 20;
    const unsigned blocks = (unsigned)(blocks_needed < max_blocks ? blocks_needed : max_blocks);
    if (dtype_bf16)
        hipLaunchKernelGGL(merge_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, o_a, lse_a,
                           o_b, lse_b, o, lse, num_rows);
    else
        hipLaunchKernelGGL(merge_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, o_a,
                           lse_a, o_b, lse_b, o, lse, num_rows);
    return hipGetLastError();
}

}  // namespace mla
