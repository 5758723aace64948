// C ABI of the MLA ragged prefill library: argument validation, plans,
// per-stream scratch for the one-shot call, and kernel dispatch.
//
// Every public function validates on the host before its first HIP call and
// returns a status; messages go to a thread-local buffer read by
// mla_last_error(). No exception escapes.
#include "../../include/mla_ragged.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

using mla::WorkItem;

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    std::string m = std::string(what) + ": " + hipGetErrorString(e);
    return fail(MLA_EHIP, m);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Pinned host staging + device buffer for one work list. Grow-only.
// A ring of pinned slots lets several uploads be in flight on a stream
// before the host has to wait for the oldest copy to finish.
//
// A buffer outgrown by a larger work list is retired, not freed: a run
// launched earlier (on this or any stream) may still read it, and HIP's
// hipFree / hipHostFree synchronise the whole device. Retired buffers are
// freed in release() (plan destruction), after the owner has waited for the
// plan's last run. Growth is geometric, so the retired buffers together stay
// smaller than the live one.
template <class Item>
struct DeviceWorkList {
    static constexpr int kRing = 4;
    Item* dev = nullptr;
    size_t dev_cap = 0;             // items
    int device = -1;
    Item* pinned[kRing] = {};
    size_t pinned_cap[kRing] = {};
    hipEvent_t done[kRing] = {};
    bool pending[kRing] = {};
    int next = 0;
    std::vector<void*> retired_dev;
    std::vector<void*> retired_pinned;

    ~DeviceWorkList() { release(); }

    // Free everything. The caller has waited for every run that reads `dev`.
    void release() {
        for (int i = 0; i < kRing; ++i) {
            if (pending[i]) (void)hipEventSynchronize(done[i]);
            if (done[i]) (void)hipEventDestroy(done[i]);
            if (pinned[i]) (void)hipHostFree(pinned[i]);
            done[i] = nullptr;
            pinned[i] = nullptr;
            pinned_cap[i] = 0;
            pending[i] = false;
        }
        for (void* p : retired_pinned) (void)hipHostFree(p);
        retired_pinned.clear();
        if (dev) (void)hipFree(dev);
        for (void* p : retired_dev) (void)hipFree(p);
        retired_dev.clear();
        dev = nullptr;
        dev_cap = 0;
    }

    static size_t grown(size_t cap, size_t need) { return need > 2 * cap ? need : 2 * cap; }

    // Asynchronously copy `items` to `dev` on `stream`. `before_release` is
    // called (with the old device current) when the list moves to another
    // device, so the owner can wait for its last run first.
    template <class Wait>
    int upload(const std::vector<Item>& items, hipStream_t stream, Wait before_release) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        if (device != -1 && device != cur) {
            // the plan moves to another device: drop the old buffers
            int keep = cur;
            (void)hipSetDevice(device);
            before_release();
            release();
            (void)hipSetDevice(keep);
        }
        device = cur;
        const size_t n = items.empty() ? 1 : items.size();
        if (dev_cap < n) {
            const size_t cap = grown(dev_cap, n);
            Item* fresh = nullptr;
            e = hipMalloc(&fresh, cap * sizeof(Item));
            if (e != hipSuccess) return fail(MLA_ENOMEM, "hipMalloc of the work list failed");
            try {
                if (dev) retired_dev.push_back(dev);
            } catch (const std::bad_alloc&) {
                (void)hipFree(fresh);
                return fail(MLA_ENOMEM, "host allocation of the retired-buffer list failed");
            }
            dev = fresh;
            dev_cap = cap;
        }
        if (items.empty()) return MLA_OK;
        const int slot = next;
        next = (next + 1) % kRing;
        if (pending[slot]) {
            // the copy four uploads ago used this slot: wait for that copy only
            e = hipEventSynchronize(done[slot]);
            if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
            pending[slot] = false;
        }
        if (pinned_cap[slot] < items.size()) {
            const size_t cap = grown(pinned_cap[slot], items.size());
            Item* fresh = nullptr;
            e = hipHostMalloc(reinterpret_cast<void**>(&fresh), cap * sizeof(Item),
                              hipHostMallocDefault);
            if (e != hipSuccess) return fail(MLA_ENOMEM, "hipHostMalloc of staging failed");
            try {
                if (pinned[slot]) retired_pinned.push_back(pinned[slot]);
            } catch (const std::bad_alloc&) {
                (void)hipHostFree(fresh);
                return fail(MLA_ENOMEM, "host allocation of the retired-buffer list failed");
            }
            pinned[slot] = fresh;
            pinned_cap[slot] = cap;
        }
        if (!done[slot]) {
            e = hipEventCreateWithFlags(&done[slot], hipEventDisableTiming);
            if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        }
        std::memcpy(pinned[slot], items.data(), items.size() * sizeof(Item));
        e = hipMemcpyAsync(dev, pinned[slot], items.size() * sizeof(Item),
                           hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync of the work list");
        e = hipEventRecord(done[slot], stream);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
        pending[slot] = true;
        return MLA_OK;
    }
};

// Completion of a plan's most recent run: recorded on the run's stream after
// its kernels, waited for (on the host) only before the plan frees memory
// that run may read. Waiting for it never waits for other work.
struct RunFence {
    hipEvent_t ev = nullptr;
    int device = -1;
    bool recorded = false;

    int record(hipStream_t stream) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        if (ev != nullptr && device != cur) {
            wait();
            (void)hipEventDestroy(ev);
            ev = nullptr;
        }
        if (ev == nullptr) {
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess) { ev = nullptr; return hip_fail(e, "hipEventCreate"); }
            device = cur;
        }
        e = hipEventRecord(ev, stream);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
        recorded = true;
        return MLA_OK;
    }
    void wait() {
        if (ev != nullptr && recorded) (void)hipEventSynchronize(ev);
        recorded = false;
    }
    ~RunFence() {
        wait();
        if (ev != nullptr) (void)hipEventDestroy(ev);
    }
};

}  // namespace

struct mla_plan {
    std::vector<WorkItem> items;
    int64_t tq = 0, tk = 0;
    int32_t batch = 0, num_heads = 0, causal = 0, dtype = -1, block_m = 0;
    int32_t n_xcd = 8;
    int32_t heads_per_item = 0;   // 0 = chosen by the planner
    int32_t items_per_wg = 1;     // work-list entries per workgroup (2: paired tiles)
    bool paged = false;           // items carry the sequence index in kv_start
    bool planned = false;
    bool uploaded = false;
    DeviceWorkList<WorkItem> dwl;
    mutable RunFence last_run;    // recorded by every run
    std::mutex oneshot_mu;        // one-shot calls sharing this (device, stream) plan
    ~mla_plan() {
        // no launched run may still read the work list when it is freed
        last_run.wait();
        dwl.release();
    }
};

struct mla_absorbed_plan {
    std::vector<mla::LatentItem> items;
    int64_t tq = 0, tk = 0, rows = 0;
    int32_t batch = 0, num_heads = 0, causal = 0, splits = 1, max_kv_len = 0;
    bool paged = false;           // items carry the sequence index in kv_start
    bool planned = false;
    bool uploaded = false;
    DeviceWorkList<mla::LatentItem> dwl;
    mutable RunFence last_run;    // recorded by every run
    std::mutex oneshot_mu;        // one-shot calls sharing this (device, stream) plan
    // fp32 partial states of the KV splits (grow-only; an outgrown buffer is
    // retired until destruction, like the work list's)
    void* part = nullptr;
    size_t part_bytes = 0;
    int part_device = -1;
    std::vector<void*> retired_part;
    void free_parts() {
        if (part != nullptr) (void)hipFree(part);
        for (void* q : retired_part) (void)hipFree(q);
        part = nullptr;
        part_bytes = 0;
        retired_part.clear();
    }
    ~mla_absorbed_plan() {
        last_run.wait();
        if (part != nullptr || !retired_part.empty()) {
            int keep = -1;
            (void)hipGetDevice(&keep);
            (void)hipSetDevice(part_device);
            free_parts();
            (void)hipSetDevice(keep);
        }
        dwl.release();
    }
};

namespace {

int check_dtype(int32_t dtype) {
    if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP32)
        return fail(MLA_EUNSUPPORTED, "dtype must be MLA_DTYPE_BF16 or MLA_DTYPE_FP32");
    return MLA_OK;
}

int check_scale(float sm_scale) {
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
        return fail(MLA_EINVAL, "sm_scale must be finite and > 0");
    return MLA_OK;
}

int check_tensors(const void* q, const void* k, const void* v, const void* out,
                  const float* lse, int64_t tq, int64_t tk) {
    if (tq > 0 && (q == nullptr || out == nullptr))
        return fail(MLA_EINVAL, "q and out must be non-NULL when there are query rows");
    if (tk > 0 && (k == nullptr || v == nullptr))
        return fail(MLA_EINVAL, "k and v must be non-NULL when there are keys");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(MLA_EINVAL, "q, k, v and out must be 16-byte aligned");
    if (!aligned16(lse) && lse != nullptr)
        return fail(MLA_EINVAL, "lse must be 16-byte aligned");
    return MLA_OK;
}

int do_plan(mla_plan* p, const int32_t* qo, const int32_t* kv, int32_t batch, int32_t heads,
            int32_t causal, int32_t dtype, bool paged = false) {
    if (p == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    p->planned = false;
    p->uploaded = false;
    if (int s = check_dtype(dtype)) return s;
    if (causal != 0 && causal != 1) return fail(MLA_EINVAL, "causal must be 0 or 1");
    if (batch < 0) return fail(MLA_EINVAL, "batch must be >= 0");
    if (heads < 1) return fail(MLA_EINVAL, "num_heads must be >= 1");
    if (batch > 0 && (qo == nullptr || kv == nullptr)) return fail(MLA_EINVAL, "indptr is NULL");
    const int bm = dtype == MLA_DTYPE_BF16 ? mla::prefill_bf16_block_m() : mla::prefill_fp32_block_m();
    // the bf16 kernel may run two work-list entries of one head each per
    // workgroup (paired light tiles); head blocks keep one entry per workgroup
    const int pair = dtype == MLA_DTYPE_BF16 && p->heads_per_item <= 1 ? mla::kPrefillPairMaxKeys : 0;
    int per_wg = 1;
    std::string err;
    try {
        if (!mla::build_work_list(qo, kv, batch, heads, causal != 0, bm, p->n_xcd,
                                  p->heads_per_item, p->items, err, paged, pair, &per_wg))
            return fail(MLA_EINVAL, err);
    } catch (const std::bad_alloc&) {
        return fail(MLA_ENOMEM, "host allocation of the work list failed");
    }
    // 32-bit token indices inside the kernels: Tq*H and Tk*H row counts must fit
    const int64_t tq = batch > 0 ? qo[batch] : 0;
    const int64_t tk = batch > 0 ? kv[batch] : 0;
    if (tq * heads > INT32_MAX || tk * heads > INT32_MAX)
        return fail(MLA_EUNSUPPORTED, "tokens x heads exceeds 2^31 rows");
    p->tq = tq;
    p->tk = tk;
    p->batch = batch;
    p->num_heads = heads;
    p->causal = causal;
    p->dtype = dtype;
    p->block_m = bm;
    p->items_per_wg = per_wg;
    p->paged = paged;
    p->planned = true;
    return MLA_OK;
}

// q_rows / kv_rows / num_heads: the sizes of the tensors the caller passes
// (kv_rows < 0: paged K/V, no contiguous key rows to check).
int do_run(const mla_plan* p, const void* q, const void* k, const void* v, int64_t q_rows,
           int64_t kv_rows, int32_t num_heads, float sm_scale, int32_t dtype, void* out,
           float* lse, hipStream_t stream, const mla::PagedKv* paged = nullptr) {
    if (p == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (p->paged != (paged != nullptr))
        return fail(MLA_ESTATE, "plan and call disagree on paged K/V");
    if (!p->planned) return fail(MLA_ESTATE, "plan has not been built");
    if (dtype != p->dtype) return fail(MLA_ESTATE, "dtype differs from the planned dtype");
    if (num_heads != p->num_heads) return fail(MLA_ESTATE, "num_heads differs from the plan");
    if (q_rows != p->tq)
        return fail(MLA_ESTATE, "q / out rows differ from the planned qo_indptr[batch]");
    if (paged == nullptr && kv_rows < p->tk)
        return fail(MLA_ESTATE, "k / v have fewer rows than the planned kv_indptr[batch]");
    if (!p->uploaded) return fail(MLA_ESTATE, "plan has not been uploaded (mla_plan_upload)");
    if (int s = check_scale(sm_scale)) return s;
    if (int s = check_tensors(q, k, v, out, lse, p->tq, paged != nullptr ? 1 : p->tk)) return s;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != p->dwl.device) return fail(MLA_ESTATE, "plan was uploaded on another device");
    if (p->items.empty()) return MLA_OK;
    const int64_t n = static_cast<int64_t>(p->items.size());
    e = dtype == MLA_DTYPE_BF16
            ? mla::launch_prefill_bf16(p->dwl.dev, n, q, k, v, out, lse, p->num_heads, sm_scale,
                                       stream, paged, p->items_per_wg)
            : mla::launch_prefill_fp32(p->dwl.dev, n, q, k, v, out, lse, p->num_heads, sm_scale,
                                       stream, paged);
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return p->last_run.record(stream);
}

// One-shot calls keep one plan per (device, stream).
std::mutex g_oneshot_mu;
std::map<std::pair<int, void*>, mla_plan*>* g_oneshot = nullptr;

// One-shot prefill (plan + upload + run) with a plan kept per (device, stream).
int oneshot(const void* q, const void* k, const void* v, const int32_t* qo_indptr,
            const int32_t* kv_indptr, int32_t batch, int32_t num_heads, int32_t causal,
            float sm_scale, int32_t dtype, void* out, float* lse, void* stream,
            const mla::PagedKv* paged) {
    // validate everything before the first HIP call
    if (int s = check_dtype(dtype)) return s;
    if (int s = check_scale(sm_scale)) return s;
    if (batch < 0) return fail(MLA_EINVAL, "batch must be >= 0");
    if (num_heads < 1) return fail(MLA_EINVAL, "num_heads must be >= 1");
    if (causal != 0 && causal != 1) return fail(MLA_EINVAL, "causal must be 0 or 1");
    if (batch > 0 && (qo_indptr == nullptr || kv_indptr == nullptr))
        return fail(MLA_EINVAL, "indptr is NULL");
    const int64_t tq = batch > 0 ? qo_indptr[batch] : 0;
    const int64_t tk = batch > 0 ? kv_indptr[batch] : 0;
    if (int s = check_tensors(q, k, v, out, lse, tq, paged != nullptr ? 1 : tk)) return s;
    mla_plan scratch_check;
    if (int s = do_plan(&scratch_check, qo_indptr, kv_indptr, batch, num_heads, causal, dtype,
                        paged != nullptr))
        return s;
    if (scratch_check.items.empty()) return MLA_OK;

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    mla_plan* p = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_oneshot_mu);
        if (g_oneshot == nullptr) g_oneshot = new (std::nothrow) std::map<std::pair<int, void*>, mla_plan*>();
        if (g_oneshot == nullptr) return fail(MLA_ENOMEM, "one-shot plan table");
        auto key = std::make_pair(dev, stream);
        auto it = g_oneshot->find(key);
        if (it == g_oneshot->end()) {
            p = new (std::nothrow) mla_plan();
            if (p == nullptr) return fail(MLA_ENOMEM, "one-shot plan");
            (*g_oneshot)[key] = p;
        } else {
            p = it->second;
        }
    }
    // The device side is ordered by the stream; threads that share the
    // stream take turns on its plan from here to the launch.
    std::lock_guard<std::mutex> plan_lock(p->oneshot_mu);
    p->items.swap(scratch_check.items);
    p->tq = scratch_check.tq;
    p->tk = scratch_check.tk;
    p->batch = batch;
    p->num_heads = num_heads;
    p->causal = causal;
    p->dtype = dtype;
    p->block_m = scratch_check.block_m;
    p->items_per_wg = scratch_check.items_per_wg;
    p->paged = scratch_check.paged;
    p->planned = true;
    p->uploaded = false;
    if (int s = mla_plan_upload(p, stream)) return s;
    return do_run(p, q, k, v, tq, paged != nullptr ? -1 : tk, num_heads, sm_scale, dtype, out,
                  lse, static_cast<hipStream_t>(stream), paged);
}

// Weight-absorbed prefill: one-shot calls keep one plan per (device, stream).
std::mutex g_absorbed_mu;
std::map<std::pair<int, void*>, mla_absorbed_plan*>* g_absorbed = nullptr;

int absorbed_plan(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t num_heads,
                  int32_t causal, std::vector<mla::LatentItem>& items, bool paged = false,
                  int* splits_out = nullptr) {
    if (causal != 0 && causal != 1) return fail(MLA_EINVAL, "causal must be 0 or 1");
    if (batch < 0) return fail(MLA_EINVAL, "batch must be >= 0");
    if (num_heads < 1) return fail(MLA_EINVAL, "num_heads must be >= 1");
    if (batch > 0 && (qo == nullptr || kv == nullptr)) return fail(MLA_EINVAL, "indptr is NULL");
    if (batch > 0 && static_cast<int64_t>(kv[batch]) * (MLA_LATENT_DIM + MLA_ROPE_DIM) > INT64_C(1) << 40)
        return fail(MLA_EUNSUPPORTED, "latent cache too large");
    std::string err;
    int splits = 1;
    if (batch > 0 && qo[0] == 0 && kv[0] == 0)
        splits = mla::latent_kv_splits(qo, kv, batch, num_heads, causal != 0,
                                       mla::prefill_absorbed_block_m());
    // the partial states of the splits stay below 1 GiB
    const int64_t rows = batch > 0 ? static_cast<int64_t>(qo[batch]) * num_heads : 0;
    while (splits > 1 && static_cast<int64_t>(splits) * rows * (MLA_LATENT_DIM + 1) * 4 > (INT64_C(1) << 30))
        --splits;
    if (splits_out != nullptr) *splits_out = splits;
    try {
        if (!mla::build_latent_work_list(qo, kv, batch, num_heads, causal != 0,
                                         mla::prefill_absorbed_block_m(), 8, items, err, paged,
                                         splits))
            return fail(MLA_EINVAL, err);
    } catch (const std::bad_alloc&) {
        return fail(MLA_ENOMEM, "host allocation of the work list failed");
    }
    return MLA_OK;
}

int absorbed_build(mla_absorbed_plan* p, const int32_t* qo, const int32_t* kv, int32_t batch,
                   int32_t num_heads, int32_t causal, bool paged) {
    if (p == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    p->planned = false;
    p->uploaded = false;
    int splits = 1;
    std::vector<mla::LatentItem> items;
    if (int s = absorbed_plan(qo, kv, batch, num_heads, causal, items, paged, &splits)) return s;
    p->items.swap(items);
    p->tq = batch > 0 ? qo[batch] : 0;
    p->tk = batch > 0 ? kv[batch] : 0;
    p->rows = p->tq * num_heads;
    p->batch = batch;
    p->num_heads = num_heads;
    p->causal = causal;
    p->splits = splits;
    p->max_kv_len = 0;
    for (int32_t b = 0; b < batch; ++b)
        p->max_kv_len = std::max<int32_t>(p->max_kv_len, kv[b + 1] - kv[b]);
    p->paged = paged;
    p->planned = true;
    return MLA_OK;
}

int absorbed_upload(mla_absorbed_plan* p, hipStream_t stream) {
    if (p == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (!p->planned) return fail(MLA_ESTATE, "plan has not been built");
    p->uploaded = false;
    if (p->items.empty()) {
        p->uploaded = true;
        return MLA_OK;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (p->splits > 1) {
        // per split and row: O in bf16, LSE in fp32
        const size_t need = static_cast<size_t>(p->splits) * static_cast<size_t>(p->rows) *
                            (MLA_LATENT_DIM * sizeof(uint16_t) + sizeof(float));
        if (p->part_device != -1 && p->part_device != dev) {
            // the plan moves to another device: its last run must end first
            p->last_run.wait();
            int keep = dev;
            (void)hipSetDevice(p->part_device);
            p->free_parts();
            (void)hipSetDevice(keep);
            p->part_device = -1;
        }
        if (p->part_bytes < need) {
            // an earlier run may still use the old buffer: retire it
            void* fresh = nullptr;
            e = hipMalloc(&fresh, need);
            if (e != hipSuccess)
                return fail(MLA_ENOMEM, "hipMalloc of the KV-split partial states failed");
            try {
                if (p->part != nullptr) p->retired_part.push_back(p->part);
            } catch (const std::bad_alloc&) {
                (void)hipFree(fresh);
                return fail(MLA_ENOMEM, "host allocation of the retired-buffer list failed");
            }
            p->part = fresh;
            p->part_bytes = need;
            p->part_device = dev;
        }
    }
    if (int r = p->dwl.upload(p->items, stream, [p] { p->last_run.wait(); })) return r;
    p->uploaded = true;
    return MLA_OK;
}

// One run of an uploaded plan (contiguous cache, or a page pool when `pg`).
// q_rows / kv_rows / num_heads: the sizes of the caller's tensors (kv_rows is
// not checked for a page pool).
int absorbed_run(const mla_absorbed_plan* p, const void* q, const void* kv, int64_t q_rows,
                 int64_t kv_rows, int32_t num_heads, float sm_scale, void* out, float* lse,
                 hipStream_t stream, const mla::PagedKv* pg) {
    if (p == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (!p->planned) return fail(MLA_ESTATE, "plan has not been built");
    if (p->paged != (pg != nullptr)) return fail(MLA_ESTATE, "plan and call disagree on paged cache");
    if (num_heads != p->num_heads) return fail(MLA_ESTATE, "num_heads differs from the plan");
    if (q_rows != p->tq)
        return fail(MLA_ESTATE, "q / out rows differ from the planned qo_indptr[batch]");
    if (pg == nullptr && kv_rows < p->tk)
        return fail(MLA_ESTATE, "kv has fewer rows than the planned kv_indptr[batch]");
    if (!p->uploaded) return fail(MLA_ESTATE, "plan has not been uploaded");
    if (int s = check_scale(sm_scale)) return s;
    if (p->tq > 0 && (q == nullptr || out == nullptr))
        return fail(MLA_EINVAL, "q and out must be non-NULL when there are query rows");
    if ((p->tk > 0 || pg != nullptr) && kv == nullptr)
        return fail(MLA_EINVAL, "kv must be non-NULL when there are keys");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (lse != nullptr && !aligned16(lse)))
        return fail(MLA_EINVAL, "q, kv, out and lse must be 16-byte aligned");
    if (pg != nullptr && p->max_kv_len > static_cast<int64_t>(pg->max_pages) * pg->page_size)
        return fail(MLA_EINVAL, "a sequence's context exceeds max_pages x page_size");
    if (p->items.empty()) return MLA_OK;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != p->dwl.device || (p->splits > 1 && dev != p->part_device))
        return fail(MLA_ESTATE, "plan was uploaded on another device");
    uint16_t* part_o = nullptr;
    float* part_lse = nullptr;
    if (p->splits > 1) {
        // the O block is splits x rows x 512 bf16 (a multiple of 1 KB), so
        // the LSE block after it stays 16-byte aligned
        part_o = static_cast<uint16_t*>(p->part);
        part_lse = reinterpret_cast<float*>(part_o + static_cast<size_t>(p->splits) * p->rows *
                                                         MLA_LATENT_DIM);
    }
    e = mla::launch_prefill_absorbed(p->dwl.dev, static_cast<int64_t>(p->items.size()), q, kv,
                                     out, lse, p->num_heads, sm_scale, stream, pg, part_o,
                                     part_lse, p->rows);
    if (e != hipSuccess) return hip_fail(e, "absorbed prefill kernel launch");
    if (p->splits > 1) {
        e = mla::launch_merge_splits(part_o, part_lse, p->splits, p->rows, out, lse, stream);
        if (e != hipSuccess) return hip_fail(e, "KV-split merge kernel launch");
    }
    return p->last_run.record(stream);
}

// One-shot absorbed call (plan + upload + run) with a plan kept per (device,
// stream); contiguous cache, or a page pool when `pg`.
int absorbed_call(const void* q, const void* kv, const int32_t* qo_indptr,
                  const int32_t* kv_indptr, int32_t batch, int32_t num_heads, int32_t causal,
                  float sm_scale, void* out, float* lse, void* stream, const mla::PagedKv* pg) {
    if (int s = check_scale(sm_scale)) return s;
    mla_absorbed_plan check;
    if (int s = absorbed_build(&check, qo_indptr, kv_indptr, batch, num_heads, causal, pg != nullptr))
        return s;
    if (check.tq > 0 && (q == nullptr || out == nullptr))
        return fail(MLA_EINVAL, "q and out must be non-NULL when there are query rows");
    if ((check.tk > 0 || pg != nullptr) && kv == nullptr)
        return fail(MLA_EINVAL, "kv must be non-NULL when there are keys");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (lse != nullptr && !aligned16(lse)))
        return fail(MLA_EINVAL, "q, kv, out and lse must be 16-byte aligned");
    if (check.items.empty()) return MLA_OK;

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    mla_absorbed_plan* p = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_absorbed_mu);
        if (g_absorbed == nullptr)
            g_absorbed = new (std::nothrow) std::map<std::pair<int, void*>, mla_absorbed_plan*>();
        if (g_absorbed == nullptr) return fail(MLA_ENOMEM, "absorbed plan table");
        auto key = std::make_pair(dev, stream);
        auto it = g_absorbed->find(key);
        if (it == g_absorbed->end()) {
            p = new (std::nothrow) mla_absorbed_plan();
            if (p == nullptr) return fail(MLA_ENOMEM, "absorbed plan");
            (*g_absorbed)[key] = p;
        } else {
            p = it->second;
        }
    }
    // the work list moves into the per-stream plan; its device buffers stay.
    // Threads that share the stream take turns on the plan up to the launch.
    std::lock_guard<std::mutex> plan_lock(p->oneshot_mu);
    p->items.swap(check.items);
    p->tq = check.tq;
    p->tk = check.tk;
    p->rows = check.rows;
    p->batch = check.batch;
    p->num_heads = check.num_heads;
    p->causal = check.causal;
    p->splits = check.splits;
    p->max_kv_len = check.max_kv_len;
    p->paged = check.paged;
    p->planned = true;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int r = absorbed_upload(p, s)) return r;
    return absorbed_run(p, q, kv, p->tq, p->tk, num_heads, sm_scale, out, lse, s, pg);
}

// Device-planned prefill: the caller's workspace, or (use_scratch) the
// library's file-scope scratch array. Validates everything on the host
// before the first HIP call; allocates nothing and makes no synchronising
// call, so it can be captured in a graph.
int device_plan_call(const void* q, const void* k, const void* v, const int32_t* qo_indptr,
                     const int32_t* kv_indptr, int32_t batch, int64_t max_tq, int64_t max_tk,
                     int32_t num_heads, int32_t causal, float sm_scale, int32_t dtype, void* out,
                     float* lse, void* workspace, int64_t workspace_bytes, bool use_scratch,
                     void* stream) {
    if (int s = check_dtype(dtype)) return s;
    if (int s = check_scale(sm_scale)) return s;
    if (batch < 0 || batch > mla::kDevicePlanMaxBatch)
        return fail(MLA_EINVAL, "batch must be in [0, 4096] for device planning");
    if (num_heads < 1 || num_heads > 65535) return fail(MLA_EINVAL, "num_heads must be in [1, 65535]");
    if (causal != 0 && causal != 1) return fail(MLA_EINVAL, "causal must be 0 or 1");
    if (max_tq < 0 || max_tk < 0) return fail(MLA_EINVAL, "max_tq and max_tk must be >= 0");
    if (max_tq * num_heads > INT32_MAX || max_tk * num_heads > INT32_MAX)
        return fail(MLA_EUNSUPPORTED, "tokens x heads exceeds 2^31 rows");
    if (batch == 0) return MLA_OK;
    if (qo_indptr == nullptr || kv_indptr == nullptr) return fail(MLA_EINVAL, "indptr is NULL");
    if (int s = check_tensors(q, k, v, out, lse, max_tq, max_tk)) return s;
    const int bm = dtype == MLA_DTYPE_BF16 ? mla::prefill_bf16_block_m() : mla::prefill_fp32_block_m();
    const int64_t n = mla::device_plan_max_items(batch, max_tq, num_heads, bm);
    const mla::DevicePlanLayout l = mla::device_plan_layout(batch, n);
    if (n > INT32_MAX) return fail(MLA_EUNSUPPORTED, "too many work items");
    if (use_scratch) {
        if (l.bytes > mla::kDevicePlanScratchBytes)
            return fail(MLA_EUNSUPPORTED,
                        "this batch needs " + std::to_string(l.bytes) +
                            " bytes of device-plan workspace; the static scratch holds " +
                            std::to_string(mla::kDevicePlanScratchBytes) +
                            " (use mla_ragged_prefill_device_plan with a workspace)");
        hipError_t e = mla::device_plan_scratch(&workspace);
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    } else {
        if (workspace == nullptr || !aligned16(workspace))
            return fail(MLA_EINVAL, "workspace must be non-NULL and 16-byte aligned");
        if (workspace_bytes < l.bytes)
            return fail(MLA_EINVAL, "workspace is smaller than mla_device_plan_workspace_size");
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = mla::launch_device_plan(qo_indptr, kv_indptr, batch, max_tq, max_tk, num_heads,
                                           causal != 0, bm, workspace, n, s);
    if (e != hipSuccess) return hip_fail(e, "device plan launch");
    const WorkItem* items =
        reinterpret_cast<const WorkItem*>(static_cast<const uint8_t*>(workspace) + l.items);
    e = dtype == MLA_DTYPE_BF16
            ? mla::launch_prefill_bf16(items, n, q, k, v, out, lse, num_heads, sm_scale, s)
            : mla::launch_prefill_fp32(items, n, q, k, v, out, lse, num_heads, sm_scale, s);
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return MLA_OK;
}

// Fused decompression + prefill: the query tiles of all sequences (one head
// each), sorted by the keys they visit, heaviest first. n_busy = tiles that
// see at least one key (a prefix of the list).
int fused_tiles(const int32_t* qo, const int32_t* kv, int32_t batch, int32_t causal,
                std::vector<WorkItem>& tiles, int64_t& n_busy) {
    std::string err;
    try {
        if (!mla::build_work_list(qo, kv, batch, 1, causal != 0, mla::decompress_prefill_block_m(),
                                  1, 1, tiles, err))
            return fail(MLA_EINVAL, err);
    } catch (const std::bad_alloc&) {
        return fail(MLA_ENOMEM, "host allocation of the work list failed");
    }
    std::stable_sort(tiles.begin(), tiles.end(),
                     [](const WorkItem& a, const WorkItem& b) { return a.kv_hi > b.kv_hi; });
    n_busy = std::count_if(tiles.begin(), tiles.end(), [](const WorkItem& t) { return t.kv_hi > 0; });
    return MLA_OK;
}

// Per (device, stream): the device copy of the tile list and the fence of
// the last run that read it.
struct FusedState {
    std::mutex mu;
    RunFence last_run;
    DeviceWorkList<WorkItem> dwl;
    ~FusedState() { last_run.wait(); }   // before the members free the list
};
std::mutex g_fused_mu;
std::map<std::pair<int, void*>, FusedState*>* g_fused = nullptr;

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "MLA_OK";
        case MLA_EINVAL: return "MLA_EINVAL";
        case MLA_EUNSUPPORTED: return "MLA_EUNSUPPORTED";
        case MLA_EHIP: return "MLA_EHIP";
        case MLA_ENOMEM: return "MLA_ENOMEM";
        case MLA_ESTATE: return "MLA_ESTATE";
        default: return "MLA_UNKNOWN_STATUS";
    }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_version(void) { return "0.1.0"; }

int mla_plan_create(mla_plan** out) {
    if (out == nullptr) return fail(MLA_EINVAL, "out is NULL");
    *out = new (std::nothrow) mla_plan();
    if (*out == nullptr) return fail(MLA_ENOMEM, "plan allocation failed");
    return MLA_OK;
}

void mla_plan_destroy(mla_plan* plan) { delete plan; }

int mla_plan_set_xcds(mla_plan* plan, int32_t n_xcd) {
    if (plan == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (n_xcd < 1 || n_xcd > 64) return fail(MLA_EINVAL, "n_xcd must be in [1, 64]");
    plan->n_xcd = n_xcd;
    return MLA_OK;
}

int mla_ragged_plan(mla_plan* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                    int32_t batch, int32_t num_heads, int32_t causal, int32_t dtype) {
    return do_plan(plan, qo_indptr, kv_indptr, batch, num_heads, causal, dtype);
}

int mla_plan_upload(mla_plan* plan, void* stream) {
    if (plan == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (!plan->planned) return fail(MLA_ESTATE, "plan has not been built");
    int s = plan->dwl.upload(plan->items, static_cast<hipStream_t>(stream),
                             [plan] { plan->last_run.wait(); });
    if (s != MLA_OK) return s;
    plan->uploaded = true;
    return MLA_OK;
}

int mla_ragged_run(const mla_plan* plan, const void* q, const void* k, const void* v,
                   int64_t q_rows, int64_t kv_rows, int32_t num_heads, float sm_scale,
                   int32_t dtype, void* out, float* lse, void* stream) {
    return do_run(plan, q, k, v, q_rows, kv_rows, num_heads, sm_scale, dtype, out, lse,
                  static_cast<hipStream_t>(stream));
}

int mla_plan_info(const mla_plan* plan, int64_t* n_items, int32_t* block_m, int32_t* n_xcd,
                  int32_t* heads_per_item) {
    if (plan == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (!plan->planned) return fail(MLA_ESTATE, "plan has not been built");
    if (n_items) *n_items = static_cast<int64_t>(plan->items.size());
    if (block_m) *block_m = plan->block_m;
    if (n_xcd) *n_xcd = plan->n_xcd;
    if (heads_per_item) {
        int32_t nh = 0;
        for (const WorkItem& w : plan->items)
            if (w.n_rows > 0) { nh = w.n_heads; break; }
        *heads_per_item = nh;
    }
    return MLA_OK;
}

int mla_plan_items_per_workgroup(const mla_plan* plan, int32_t* items_per_workgroup) {
    if (plan == nullptr || items_per_workgroup == nullptr)
        return fail(MLA_EINVAL, "plan or items_per_workgroup is NULL");
    if (!plan->planned) return fail(MLA_ESTATE, "plan has not been built");
    *items_per_workgroup = plan->items_per_wg;
    return MLA_OK;
}

int mla_plan_set_heads_per_item(mla_plan* plan, int32_t heads_per_item) {
    if (plan == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (heads_per_item < 0) return fail(MLA_EINVAL, "heads_per_item must be >= 0");
    plan->heads_per_item = heads_per_item;
    return MLA_OK;
}

int mla_plan_items(const mla_plan* plan, int32_t* dst, int64_t capacity_items) {
    if (plan == nullptr || dst == nullptr) return fail(MLA_EINVAL, "plan or dst is NULL");
    if (!plan->planned) return fail(MLA_ESTATE, "plan has not been built");
    if (capacity_items < static_cast<int64_t>(plan->items.size()))
        return fail(MLA_EINVAL, "capacity is smaller than the item count");
    if (!plan->items.empty())
        std::memcpy(dst, plan->items.data(), plan->items.size() * sizeof(WorkItem));
    return MLA_OK;
}

int mla_ragged_prefill(const void* q, const void* k, const void* v, const int32_t* qo_indptr,
                       const int32_t* kv_indptr, int32_t batch, int32_t num_heads,
                       int32_t causal, float sm_scale, int32_t dtype, void* out, float* lse,
                       void* stream) {
    return oneshot(q, k, v, qo_indptr, kv_indptr, batch, num_heads, causal, sm_scale, dtype, out,
                   lse, stream, nullptr);
}

int mla_ragged_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* block_table, int32_t max_pages, int32_t page_size,
                             int32_t num_pages, int32_t batch, int32_t num_heads, int32_t causal,
                             float sm_scale, int32_t dtype, void* out, float* lse, void* stream) {
    if (page_size < 32 || page_size % 32 != 0)
        return fail(MLA_EINVAL, "page_size must be a positive multiple of 32");
    if (max_pages < 1 || num_pages < 1) return fail(MLA_EINVAL, "max_pages and num_pages must be >= 1");
    if ((int64_t)num_pages * page_size * (int64_t)(num_heads > 0 ? num_heads : 1) > INT32_MAX)
        return fail(MLA_EUNSUPPORTED, "cache tokens x heads exceeds 2^31 rows");
    if (batch > 0 && (block_table == nullptr ||
                      (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0))
        return fail(MLA_EINVAL, "block_table must be non-NULL and 4-byte aligned");
    if (batch > 0 && kv_indptr != nullptr) {
        for (int32_t b = 0; b < batch; ++b) {
            const int64_t len = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
            if (len > (int64_t)max_pages * page_size)
                return fail(MLA_EINVAL, "a sequence's context exceeds max_pages x page_size");
        }
    }
    const mla::PagedKv pg{block_table, max_pages, page_size, num_pages};
    return oneshot(q, k_cache, v_cache, qo_indptr, kv_indptr, batch, num_heads, causal, sm_scale,
                   dtype, out, lse, stream, &pg);
}

int mla_device_plan_workspace_size(int32_t batch, int64_t max_tq, int32_t num_heads,
                                   int32_t dtype, int64_t* bytes) {
    if (bytes == nullptr) return fail(MLA_EINVAL, "bytes is NULL");
    *bytes = 0;
    if (int s = check_dtype(dtype)) return s;
    if (batch < 0 || batch > mla::kDevicePlanMaxBatch)
        return fail(MLA_EINVAL, "batch must be in [0, 4096] for device planning");
    if (num_heads < 1 || num_heads > 65535) return fail(MLA_EINVAL, "num_heads must be in [1, 65535]");
    if (max_tq < 0) return fail(MLA_EINVAL, "max_tq must be >= 0");
    const int bm = dtype == MLA_DTYPE_BF16 ? mla::prefill_bf16_block_m() : mla::prefill_fp32_block_m();
    const int64_t n = mla::device_plan_max_items(batch, max_tq, num_heads, bm);
    *bytes = mla::device_plan_layout(batch, n).bytes;
    return MLA_OK;
}

int mla_ragged_prefill_device_plan(const void* q, const void* k, const void* v,
                                   const int32_t* qo_indptr, const int32_t* kv_indptr,
                                   int32_t batch, int64_t max_tq, int64_t max_tk,
                                   int32_t num_heads, int32_t causal, float sm_scale,
                                   int32_t dtype, void* out, float* lse, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
    return device_plan_call(q, k, v, qo_indptr, kv_indptr, batch, max_tq, max_tk, num_heads,
                            causal, sm_scale, dtype, out, lse, workspace, workspace_bytes, false,
                            stream);
}

int mla_ragged_prefill_device_plan_noalloc(const void* q, const void* k, const void* v,
                                           const int32_t* qo_indptr, const int32_t* kv_indptr,
                                           int32_t batch, int64_t max_tq, int64_t max_tk,
                                           int32_t num_heads, int32_t causal, float sm_scale,
                                           int32_t dtype, void* out, float* lse, void* stream) {
    return device_plan_call(q, k, v, qo_indptr, kv_indptr, batch, max_tq, max_tk, num_heads,
                            causal, sm_scale, dtype, out, lse, nullptr, 0, true, stream);
}

int mla_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o, float* lse, int64_t num_rows, int32_t head_dim, int32_t dtype,
                    void* stream) {
    if (int s = check_dtype(dtype)) return s;
    if (head_dim != MLA_HEAD_DIM_VO) return fail(MLA_EUNSUPPORTED, "head_dim must be 128");
    if (num_rows < 0) return fail(MLA_EINVAL, "num_rows must be >= 0");
    if (num_rows == 0) return MLA_OK;
    if (num_rows > INT32_MAX) return fail(MLA_EUNSUPPORTED, "num_rows exceeds 2^31");
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse)
        return fail(MLA_EINVAL, "merge_state pointers must be non-NULL");
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o) || !aligned16(lse_a) ||
        !aligned16(lse_b) || !aligned16(lse))
        return fail(MLA_EINVAL, "merge_state pointers must be 16-byte aligned");
    hipError_t e = mla::launch_merge(o_a, lse_a, o_b, lse_b, o, lse, num_rows,
                                     dtype == MLA_DTYPE_BF16 ? 1 : 0,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return MLA_OK;
}

int mla_decompress_kv(const void* c_kv, const void* k_rope, const void* w_uk, const void* w_uv,
                      int64_t num_tokens, int32_t num_heads, void* k_out, void* v_out,
                      void* stream) {
    if (num_tokens < 0) return fail(MLA_EINVAL, "num_tokens must be >= 0");
    if (num_heads < 1) return fail(MLA_EINVAL, "num_heads must be >= 1");
    if (num_tokens == 0) return MLA_OK;
    if (num_tokens * num_heads > INT32_MAX)
        return fail(MLA_EUNSUPPORTED, "tokens x heads exceeds 2^31 rows");
    if (!c_kv || !k_rope || !w_uk || !w_uv || !k_out || !v_out)
        return fail(MLA_EINVAL, "decompression pointers must be non-NULL");
    if (!aligned16(c_kv) || !aligned16(k_rope) || !aligned16(w_uk) || !aligned16(w_uv) ||
        !aligned16(k_out) || !aligned16(v_out))
        return fail(MLA_EINVAL, "decompression pointers must be 16-byte aligned");
    hipError_t e = mla::launch_decompress(c_kv, k_rope, w_uk, w_uv, num_tokens, num_heads, k_out,
                                          v_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decompression kernel launch");
    return MLA_OK;
}

int mla_decompress_prefill(const void* q, const void* c_kv, const void* k_rope, const void* w_uk,
                           const void* w_uv, const int32_t* qo_indptr, const int32_t* kv_indptr,
                           int32_t batch, int32_t num_heads, int32_t causal, float sm_scale,
                           void* out, float* lse, void* stream) {
    if (int s = check_scale(sm_scale)) return s;
    if (batch < 0) return fail(MLA_EINVAL, "batch must be >= 0");
    if (num_heads < 1 || num_heads > 65535) return fail(MLA_EINVAL, "num_heads must be in [1, 65535]");
    if (causal != 0 && causal != 1) return fail(MLA_EINVAL, "causal must be 0 or 1");
    if (batch > 0 && (qo_indptr == nullptr || kv_indptr == nullptr))
        return fail(MLA_EINVAL, "indptr is NULL");
    std::vector<WorkItem> tiles;
    int64_t n_busy = 0;
    if (int s = fused_tiles(qo_indptr, kv_indptr, batch, causal, tiles, n_busy)) return s;
    const int64_t tq = batch > 0 ? qo_indptr[batch] : 0;
    const int64_t tk = batch > 0 ? kv_indptr[batch] : 0;
    if (tq * num_heads > INT32_MAX || tk * num_heads > INT32_MAX)
        return fail(MLA_EUNSUPPORTED, "tokens x heads exceeds 2^31 rows");
    if (tq > 0 && (q == nullptr || out == nullptr))
        return fail(MLA_EINVAL, "q and out must be non-NULL when there are query rows");
    if (n_busy > 0 && (!c_kv || !k_rope || !w_uk || !w_uv))
        return fail(MLA_EINVAL, "c_kv, k_rope, w_uk and w_uv must be non-NULL when keys are visible");
    if (!aligned16(q) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(w_uk) ||
        !aligned16(w_uv) || !aligned16(out) || (lse != nullptr && !aligned16(lse)))
        return fail(MLA_EINVAL, "all device pointers must be 16-byte aligned");
    if (tiles.empty()) return MLA_OK;

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    FusedState* st = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_fused_mu);
        if (g_fused == nullptr) g_fused = new (std::nothrow) std::map<std::pair<int, void*>, FusedState*>();
        if (g_fused == nullptr) return fail(MLA_ENOMEM, "fused state table");
        auto key = std::make_pair(dev, stream);
        auto it = g_fused->find(key);
        if (it == g_fused->end()) {
            st = new (std::nothrow) FusedState();
            if (st == nullptr) return fail(MLA_ENOMEM, "fused state");
            (*g_fused)[key] = st;
        } else {
            st = it->second;
        }
    }
    // threads that share the stream take turns from the upload to the launch
    std::lock_guard<std::mutex> state_lock(st->mu);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int r = st->dwl.upload(tiles, s, [st] { st->last_run.wait(); })) return r;
    e = mla::launch_decompress_prefill(st->dwl.dev, static_cast<int64_t>(tiles.size()), n_busy, q,
                                       c_kv, k_rope, w_uk, w_uv, out, lse, num_heads, sm_scale, s);
    if (e != hipSuccess) return hip_fail(e, "fused decompression + prefill kernel launch");
    return st->last_run.record(s);
}

int mla_absorbed_plan_items(const int32_t* qo_indptr, const int32_t* kv_indptr, int32_t batch,
                            int32_t num_heads, int32_t causal, int32_t* dst,
                            int64_t capacity_items, int64_t* n_items) {
    if (n_items == nullptr) return fail(MLA_EINVAL, "n_items is NULL");
    std::vector<mla::LatentItem> items;
    if (int s = absorbed_plan(qo_indptr, kv_indptr, batch, num_heads, causal, items)) return s;
    *n_items = static_cast<int64_t>(items.size());
    if (dst == nullptr) return MLA_OK;
    if (capacity_items < static_cast<int64_t>(items.size()))
        return fail(MLA_EINVAL, "capacity too small for the work list");
    if (!items.empty()) std::memcpy(dst, items.data(), items.size() * sizeof(mla::LatentItem));
    static_assert(sizeof(mla::LatentItem) == 12 * sizeof(int32_t), "12 int32 per item");
    return MLA_OK;
}

int mla_absorbed_plan_create(mla_absorbed_plan** out) {
    if (out == nullptr) return fail(MLA_EINVAL, "out is NULL");
    *out = new (std::nothrow) mla_absorbed_plan();
    if (*out == nullptr) return fail(MLA_ENOMEM, "absorbed plan");
    return MLA_OK;
}

void mla_absorbed_plan_destroy(mla_absorbed_plan* plan) { delete plan; }

int mla_absorbed_plan_build(mla_absorbed_plan* plan, const int32_t* qo_indptr,
                            const int32_t* kv_indptr, int32_t batch, int32_t num_heads,
                            int32_t causal, int32_t paged) {
    if (paged != 0 && paged != 1) return fail(MLA_EINVAL, "paged must be 0 or 1");
    return absorbed_build(plan, qo_indptr, kv_indptr, batch, num_heads, causal, paged != 0);
}

int mla_absorbed_plan_upload(mla_absorbed_plan* plan, void* stream) {
    return absorbed_upload(plan, static_cast<hipStream_t>(stream));
}

int mla_absorbed_run(const mla_absorbed_plan* plan, const void* q, const void* kv,
                     int64_t q_rows, int64_t kv_rows, int32_t num_heads, float sm_scale,
                     void* out, float* lse, void* stream) {
    return absorbed_run(plan, q, kv, q_rows, kv_rows, num_heads, sm_scale, out, lse,
                        static_cast<hipStream_t>(stream), nullptr);
}

int mla_absorbed_run_paged(const mla_absorbed_plan* plan, const void* q, const void* kv_cache,
                           int64_t q_rows, int32_t num_heads, const int32_t* block_table,
                           int32_t max_pages, int32_t page_size, int32_t num_pages,
                           float sm_scale, void* out, float* lse, void* stream) {
    if (page_size < 32 || page_size % 32 != 0)
        return fail(MLA_EINVAL, "page_size must be a positive multiple of 32");
    if (max_pages < 1 || num_pages < 1) return fail(MLA_EINVAL, "max_pages and num_pages must be >= 1");
    if (plan != nullptr && plan->batch > 0 &&
        (block_table == nullptr || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0))
        return fail(MLA_EINVAL, "block_table must be non-NULL and 4-byte aligned");
    const mla::PagedKv pg{block_table, max_pages, page_size, num_pages};
    return absorbed_run(plan, q, kv_cache, q_rows, -1, num_heads, sm_scale, out, lse,
                        static_cast<hipStream_t>(stream), &pg);
}

int mla_absorbed_plan_info(const mla_absorbed_plan* plan, int64_t* n_items, int32_t* splits) {
    if (plan == nullptr) return fail(MLA_EINVAL, "plan is NULL");
    if (!plan->planned) return fail(MLA_ESTATE, "plan has not been built");
    if (n_items != nullptr) *n_items = static_cast<int64_t>(plan->items.size());
    if (splits != nullptr) *splits = plan->splits;
    return MLA_OK;
}

int mla_absorbed_prefill(const void* q, const void* kv, const int32_t* qo_indptr,
                         const int32_t* kv_indptr, int32_t batch, int32_t num_heads,
                         int32_t causal, float sm_scale, void* out, float* lse, void* stream) {
    return absorbed_call(q, kv, qo_indptr, kv_indptr, batch, num_heads, causal, sm_scale, out, lse,
                         stream, nullptr);
}

int mla_absorbed_prefill_paged(const void* q, const void* kv_cache, const int32_t* qo_indptr,
                               const int32_t* kv_indptr, const int32_t* block_table,
                               int32_t max_pages, int32_t page_size, int32_t num_pages,
                               int32_t batch, int32_t num_heads, int32_t causal, float sm_scale,
                               void* out, float* lse, void* stream) {
    if (page_size < 32 || page_size % 32 != 0)
        return fail(MLA_EINVAL, "page_size must be a positive multiple of 32");
    if (max_pages < 1 || num_pages < 1) return fail(MLA_EINVAL, "max_pages and num_pages must be >= 1");
    if (batch > 0 && (block_table == nullptr ||
                      (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0))
        return fail(MLA_EINVAL, "block_table must be non-NULL and 4-byte aligned");
    if (batch > 0 && kv_indptr != nullptr) {
        for (int32_t b = 0; b < batch; ++b) {
            const int64_t len = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
            if (len > (int64_t)max_pages * page_size)
                return fail(MLA_EINVAL, "a sequence's context exceeds max_pages x page_size");
        }
    }
    const mla::PagedKv pg{block_table, max_pages, page_size, num_pages};
    return absorbed_call(q, kv_cache, qo_indptr, kv_indptr, batch, num_heads, causal, sm_scale,
                         out, lse, stream, &pg);
}

}  // extern "C"
