// Ragged MLA prefill attention, fp32 inputs, for gfx950.
//
// Same definition as the bf16 kernel (ragged prefill with LSE,
// "vllm.v1.attention.backends.mla.prefill.flashinfer", run() with
// return_lse; head dims 192 / 128 from sglang issue 3849) computed entirely
// in fp32 FMA arithmetic, so fp32 inputs are not rounded to bf16. It serves
// accuracy (fp32 callers, the 1e-4 / 1e-5 bounds); the bf16 MFMA kernel is
// the throughput path.
//
// One wave per work item (its heads one after the other), one query row per
// lane (64-row tiles). K and V
// tiles of 32 keys are staged in LDS and read as broadcasts (all lanes read
// the same key), scores for the tile are kept in registers, then one
// online-softmax update per tile.
#include "internal.h"

namespace mla {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64;
constexpr int kBN = 32;
constexpr float kLn2 = 0.6931471805599453f;

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void prefill_fp32_kernel(
    const WorkItem* __restrict__ items, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, float* __restrict__ out, float* __restrict__ lse, int num_heads,
    float scale_log2, PagedKv pg) {
    __shared__ __attribute__((aligned(16))) float ks[kBN][kDqk];
    __shared__ __attribute__((aligned(16))) float vs[kBN][kDvo];

    const WorkItem it = items[blockIdx.x];
    if (it.n_rows <= 0) return;
    const int lane = threadIdx.x;
    const int H = num_heads;
    const bool valid = lane < it.n_rows;

    int lim = it.diag0 + lane + 1;
    lim = lim < 0 ? 0 : (lim > it.kv_len ? it.kv_len : lim);

    for (int head = it.head0; head < it.head0 + it.n_heads; ++head) {
        float qv[kDqk];
        const int64_t qrow = (int64_t)(it.q_row0 + lane) * H + head;
#pragma unroll
        for (int d = 0; d < kDqk; d += 4) {
            f32x4_t x = valid ? *reinterpret_cast<const f32x4_t*>(q + qrow * kDqk + d) : f32x4_t{};
            qv[d] = x[0]; qv[d + 1] = x[1]; qv[d + 2] = x[2]; qv[d + 3] = x[3];
        }
        float o[kDvo];
#pragma unroll
        for (int d = 0; d < kDvo; ++d) o[d] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        // K/V row (token index in the cache, head 0) of key `key`
        auto kv_row = [&](int key) -> int64_t {
            if constexpr (kPaged) {
                int pgi = pg.block_table[(int64_t)it.kv_start * pg.max_pages + key / pg.page_size];
                pgi = pgi < 0 ? 0 : (pgi >= pg.num_pages ? pg.num_pages - 1 : pgi);
                return ((int64_t)pgi * pg.page_size + key % pg.page_size) * H;
            } else {
                return ((int64_t)it.kv_start + key) * H;
            }
        };

        for (int key0 = 0; key0 < it.kv_hi; key0 += kBN) {
            __syncthreads();
            for (int u = lane; u < kBN * (kDqk / 4); u += kThreads) {
                const int row = u / (kDqk / 4), c = u % (kDqk / 4);
                const int key = key0 + row;
                *reinterpret_cast<f32x4_t*>(&ks[row][c * 4]) =
                    key < it.kv_len ? *reinterpret_cast<const f32x4_t*>(k + (kv_row(key) + head) * kDqk + c * 4)
                                    : f32x4_t{};
            }
            for (int u = lane; u < kBN * (kDvo / 4); u += kThreads) {
                const int row = u / (kDvo / 4), c = u % (kDvo / 4);
                const int key = key0 + row;
                *reinterpret_cast<f32x4_t*>(&vs[row][c * 4]) =
                    key < it.kv_len ? *reinterpret_cast<const f32x4_t*>(v + (kv_row(key) + head) * kDvo + c * 4)
                                    : f32x4_t{};
            }
            __syncthreads();

            float s[kBN];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < kBN; ++j) {
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < kDqk; ++d) dot = __builtin_fmaf(qv[d], ks[j][d], dot);
                s[j] = key0 + j < lim ? dot * scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[j]);
            }
            const float m_new = fmaxf(m_run, mx);
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - msub);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < kDvo; ++d) o[d] *= alpha;
#pragma unroll
            for (int j = 0; j < kBN; ++j) {
                const float p = __builtin_amdgcn_exp2f(s[j] - msub);
                l_run += p;
#pragma unroll
                for (int d = 0; d < kDvo; ++d) o[d] = __builtin_fmaf(p, vs[j][d], o[d]);
            }
        }

        if (!valid) continue;
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
        for (int d = 0; d < kDvo; d += 4) {
            f32x4_t x = {o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv};
            *reinterpret_cast<f32x4_t*>(out + qrow * kDvo + d) = x;
        }
        if (lse != nullptr) lse[qrow] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    }
}

}  // namespace

int prefill_fp32_block_m() { return kThreads; }

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
