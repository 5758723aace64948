// Host-only driver for the address/undefined-behaviour sanitizer test: runs
// the work partitioners and the C ABI's host paths (validation, planning,
// plan inspection) over seeded random ragged batches, including invalid
// inputs. No function here reaches a HIP call: the kernel launchers are
// stubbed out and the entry points exercised all return before any device
// work.
#include <cstdio>
#include <random>
#include <string>
#include <vector>

#include "../../include/mla_ragged.h"
#include "../../mla_ragged_chunked_amd/csrc/internal.h"

namespace mla {
// stand-ins for the kernel launchers, which live in the HIP sources
int prefill_bf16_block_m() { return 128; }
int prefill_fp32_block_m() { return 64; }
int prefill_absorbed_block_m() { return 128; }
hipError_t launch_prefill_bf16(const WorkItem*, int64_t, const void*, const void*, const void*,
                               void*, float*, int, float, hipStream_t, const PagedKv*, int) {
    return hipErrorInvalidValue;
}
hipError_t launch_prefill_fp32(const WorkItem*, int64_t, const void*, const void*, const void*,
                               void*, float*, int, float, hipStream_t, const PagedKv*) {
    return hipErrorInvalidValue;
}
hipError_t launch_prefill_absorbed(const LatentItem*, int64_t, const void*, const void*, void*,
                                   float*, int, float, hipStream_t, const PagedKv*, uint16_t*, float*,
                                   int64_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_merge_splits(const uint16_t*, const float*, int, int64_t, void*, float*,
                               hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_merge(const void*, const float*, const void*, const float*, void*, float*,
                        int64_t, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_decompress(const void*, const void*, const void*, const void*, int64_t, int,
                             void*, void*, hipStream_t) {
    return hipErrorInvalidValue;
}
int decompress_prefill_block_m() { return 128; }
hipError_t launch_decompress_prefill(const WorkItem*, int64_t, int64_t, const void*, const void*,
                                     const void*, const void*, const void*, void*, float*, int,
                                     float, hipStream_t) {
    return hipErrorInvalidValue;
}
int64_t device_plan_max_items(int batch, int64_t max_tq, int num_heads, int block_m) {
    return 8LL * ((num_heads + 7) / 8) * ((max_tq + block_m - 1) / block_m + batch);
}
DevicePlanLayout device_plan_layout(int batch, int64_t max_items) {
    DevicePlanLayout l{0, 256, 512, 1024, 1024 + max_items * 32};
    (void)batch;
    return l;
}
hipError_t launch_device_plan(const int32_t*, const int32_t*, int, int64_t, int64_t, int, bool,
                              int, void*, int64_t, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t device_plan_scratch(void**) { return hipErrorInvalidValue; }
}  // namespace mla

int main() {
    std::mt19937 rng(1234);
    int checks = 0;
    for (int trial = 0; trial < 300; ++trial) {
        const int batch = static_cast<int>(rng() % 9);
        std::vector<int32_t> qo(batch + 1, 0), kv(batch + 1, 0);
        for (int b = 0; b < batch; ++b) {
            const int q = (rng() % 5 == 0) ? 0 : static_cast<int>(rng() % 700);
            const int k = (rng() % 7 == 0) ? 0 : static_cast<int>(rng() % 1300);
            qo[b + 1] = qo[b] + q;
            kv[b + 1] = kv[b] + k;
        }
        for (int heads : {1, 3, 16, 128}) {
            for (int causal = 0; causal < 2; ++causal) {
                std::vector<mla::WorkItem> w;
                std::vector<mla::LatentItem> l;
                std::string err;
                checks += mla::build_work_list(qo.data(), kv.data(), batch, heads, causal, 128, 8,
                                               0, w, err);
                checks += mla::build_work_list(qo.data(), kv.data(), batch, heads, causal, 64, 1,
                                               heads % 2 == 0 ? 2 : 1, w, err, true);
                int per_wg = 0;
                checks += mla::build_work_list(qo.data(), kv.data(), batch, heads, causal, 128, 8,
                                               0, w, err, trial % 2 == 0, 512, &per_wg);
                checks += w.size() % (8 * static_cast<size_t>(per_wg)) == 0;
                const int s = mla::latent_kv_splits(qo.data(), kv.data(), batch, heads, causal,
                                                    128);
                checks += mla::build_latent_work_list(qo.data(), kv.data(), batch, heads, causal,
                                                      128, 8, l, err, false, s);
                checks += mla::build_latent_work_list(qo.data(), kv.data(), batch, heads, causal,
                                                      128, 8, l, err, true, 3);
                // the C ABI's host paths
                int64_t n = 0;
                checks += mla_absorbed_plan_items(qo.data(), kv.data(), batch, heads, causal,
                                                  nullptr, 0, &n) == MLA_OK;
                std::vector<int32_t> buf(static_cast<size_t>(n) * 12 + 12);
                checks += mla_absorbed_plan_items(qo.data(), kv.data(), batch, heads, causal,
                                                  buf.data(), n, &n) == MLA_OK;
                mla_plan* p = nullptr;
                checks += mla_plan_create(&p) == MLA_OK;
                checks += mla_ragged_plan(p, qo.data(), kv.data(), batch, heads, causal,
                                          MLA_DTYPE_BF16) == MLA_OK;
                int64_t items = 0;
                int32_t bm = 0, nx = 0, hpi = 0;
                checks += mla_plan_info(p, &items, &bm, &nx, &hpi) == MLA_OK;
                std::vector<int32_t> wbuf(static_cast<size_t>(items) * 8 + 8);
                checks += mla_plan_items(p, wbuf.data(), items) == MLA_OK;
                int32_t ipw = 0;
                checks += mla_plan_items_per_workgroup(p, &ipw) == MLA_OK && (ipw == 1 || ipw == 2);
                mla_plan_destroy(p);
                mla_absorbed_plan* ap = nullptr;
                checks += mla_absorbed_plan_create(&ap) == MLA_OK;
                checks += mla_absorbed_plan_build(ap, qo.data(), kv.data(), batch, heads, causal,
                                                  trial % 2) == MLA_OK;
                int32_t splits = 0;
                checks += mla_absorbed_plan_info(ap, &n, &splits) == MLA_OK;
                // not uploaded (or built for a page pool): a state error
                checks += mla_absorbed_run(ap, nullptr, nullptr, batch > 0 ? qo[batch] : 0,
                                           batch > 0 ? kv[batch] : 0, heads, 0.1f, nullptr,
                                           nullptr, nullptr) == MLA_ESTATE;
                // sizes that do not match the plan: a state error too
                checks += mla_absorbed_run(ap, nullptr, nullptr, -1, 0, heads, 0.1f, nullptr,
                                           nullptr, nullptr) == MLA_ESTATE;
                mla_absorbed_plan_destroy(ap);
            }
        }
    }
    // invalid inputs must be rejected with a status, before any HIP call
    std::vector<int32_t> bad_qo = {0, 5, 3}, ok_kv = {0, 4, 8}, nonzero = {1, 5, 9};
    std::vector<mla::WorkItem> w;
    std::vector<mla::LatentItem> l;
    std::string err;
    checks += !mla::build_work_list(bad_qo.data(), ok_kv.data(), 2, 4, true, 128, 8, 0, w, err);
    checks += !mla::build_latent_work_list(bad_qo.data(), ok_kv.data(), 2, 4, true, 128, 8, l, err);
    checks += !mla::build_latent_work_list(nonzero.data(), ok_kv.data(), 2, 4, true, 128, 8, l, err);
    checks += !mla::build_latent_work_list(ok_kv.data(), ok_kv.data(), -1, 4, true, 128, 8, l, err);
    checks += !mla::build_latent_work_list(ok_kv.data(), ok_kv.data(), 2, 4, true, 128, 8, l, err,
                                           false, 0);
    checks += mla_ragged_prefill(nullptr, nullptr, nullptr, bad_qo.data(), ok_kv.data(), 2, 4, 1,
                                 0.1f, MLA_DTYPE_BF16, nullptr, nullptr, nullptr) != MLA_OK;
    checks += mla_absorbed_prefill(nullptr, nullptr, bad_qo.data(), ok_kv.data(), 2, 4, 1, 0.1f,
                                   nullptr, nullptr, nullptr) != MLA_OK;
    checks += mla_merge_state(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 10, 128,
                              MLA_DTYPE_BF16, nullptr) != MLA_OK;
    checks += mla_decompress_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, bad_qo.data(),
                                     ok_kv.data(), 2, 4, 1, 0.1f, nullptr, nullptr,
                                     nullptr) == MLA_EINVAL;
    checks += mla_decompress_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, ok_kv.data(),
                                     ok_kv.data(), 2, 4, 1, 0.1f, nullptr, nullptr,
                                     nullptr) == MLA_EINVAL;   // NULL tensors
    // the allocation-free device plan: oversize and invalid calls fail on the host
    static int32_t dummy[64];
    checks += mla_ragged_prefill_device_plan_noalloc(dummy, dummy, dummy, ok_kv.data(),
                                                     ok_kv.data(), 2, 1000000, 1000000, 128, 1,
                                                     0.1f, MLA_DTYPE_BF16, dummy, nullptr,
                                                     nullptr) == MLA_EUNSUPPORTED;
    checks += mla_ragged_prefill_device_plan_noalloc(dummy, dummy, dummy, ok_kv.data(),
                                                     ok_kv.data(), 2, 8, 8, 0, 1, 0.1f,
                                                     MLA_DTYPE_BF16, dummy, nullptr,
                                                     nullptr) == MLA_EINVAL;
    std::printf("sanitize driver: %d checks passed\n", checks);
    return 0;
}
