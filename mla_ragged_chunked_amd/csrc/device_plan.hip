// Device-side work partitioner: builds the prefill work list on the GPU from
// device-resident indptrs, into a caller-provided workspace, so a whole
// prefill call (plan + run) can be enqueued, or captured in a HIP graph,
// with no host synchronisation and no allocation. The pages plan on the host
// once per batch ("vllm.v1.attention.backends.mla.prefill.flashinfer",
// plan() inside finalize_attention_metadata); serving loops that replay
// captured graphs need the plan to follow the indptrs on the device instead,
// in buffers whose addresses stay fixed across replays (as the metadata
// builder of "vllm/models/deepseek_v4/sparse_mla.py" pre-allocates its
// metadata buffers in __init__ for CUDA-graph address stability).
//
// Order (same goals as the host partitioner, simpler rule):
//  * Sequences are sorted by cost, heaviest first (cost of a sequence = sum
//    over its query tiles of the keys the tile visits plus a fixed charge).
//  * XCD x (workgroup i runs on XCD i % 8) takes the heads h with h % 8 == x:
//    with 8 | H every XCD gets exactly the same work. Its queue lists, in
//    sequence order, each of its heads with all that head's query tiles,
//    heaviest tile first, so the tiles that share K/V run together on one
//    XCD's L2.
//  * The grid is sized from upper bounds (max_tq, batch), so it does not
//    depend on the indptr values; unused slots are padding items.
// Invalid device indptrs (decreasing, negative, or beyond max_tq / max_tk)
// turn the offending sequence into no work, and set a flag word in the
// workspace, so a bad input can neither fault nor read out of bounds.
#include <map>
#include <mutex>

#include "internal.h"

namespace mla {

// Workspace of the allocation-free entry point: a file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// In host code `scratch` is only a stand-in for the symbol, never a device
// address: device_plan_scratch() resolves the array's address on the
// current device and every kernel argument uses that address.
__device__ __align__(256) uint8_t scratch[kDevicePlanScratchBytes];

namespace {

constexpr int kSortThreads = 1024;
constexpr int kItemThreads = 256;
constexpr int kTileCharge = 64;   // Q load + epilogue, in key-equivalents (as on the host)

__global__ __launch_bounds__(kSortThreads) void dplan_order_kernel(
    const int32_t* __restrict__ qo, const int32_t* __restrict__ kv, int batch, int64_t max_tq,
    int64_t max_tk, int causal, int block_m, int32_t* __restrict__ flag,
    int32_t* __restrict__ order, int32_t* __restrict__ prefix) {
    __shared__ uint64_t keys[kDevicePlanMaxBatch];
    __shared__ int32_t tiles_of[kDevicePlanMaxBatch];
    __shared__ int32_t part[kSortThreads];
    __shared__ int bad;
    const int tid = threadIdx.x;
    if (tid == 0) bad = (qo[0] != 0 || kv[0] != 0) ? 1 : 0;
    int n = 1;
    while (n < batch) n <<= 1;
    __syncthreads();

    // per-sequence tiles and cost; key sorts ascending = heaviest first,
    // then lower index; padding keys (all ones) sort last
    for (int b = tid; b < n; b += kSortThreads) {
        uint64_t key = ~0ull;
        if (b < batch) {
            const int64_t q0 = qo[b], q1 = qo[b + 1], k0 = kv[b], k1 = kv[b + 1];
            const bool ok = q0 >= 0 && q1 >= q0 && q1 <= max_tq && k0 >= 0 && k1 >= k0 && k1 <= max_tk;
            int tl = 0;
            int64_t cost = 0;
            if (ok) {
                const int64_t qo_len = q1 - q0, kv_len = k1 - k0;
                tl = (int)((qo_len + block_m - 1) / block_m);
                for (int t = 0; t < tl; ++t) {
                    const int64_t r0 = (int64_t)t * block_m;
                    const int64_t rows = qo_len - r0 < block_m ? qo_len - r0 : block_m;
                    const int64_t diag0 = causal ? kv_len - qo_len + r0 : kv_len;
                    int64_t hi = diag0 + rows;
                    hi = hi < 0 ? 0 : (hi > kv_len ? kv_len : hi);
                    cost += hi + kTileCharge;
                }
            } else {
                atomicOr(&bad, 1);
            }
            tiles_of[b] = tl;
            const uint64_t c = cost > 0x7fffffffLL ? 0x7fffffffull : (uint64_t)cost;
            key = ((0x7fffffffull - c) << 12) | (uint64_t)b;
        }
        keys[b] = key;
    }
    __syncthreads();

    // bitonic sort of n keys in LDS
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n; i += kSortThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const bool up = (i & k) == 0;
                    const uint64_t a = keys[i], c = keys[ixj];
                    if ((a > c) == up) {
                        keys[i] = c;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }

    // order and exclusive prefix of tiles in sorted order; each thread owns
    // a run of consecutive ranks
    const int per = (batch + kSortThreads - 1) / kSortThreads;   // <= 4
    const int r_begin = tid * per;
    int sum = 0;
    for (int r = r_begin; r < r_begin + per && r < batch; ++r) {
        const int b = (int)(keys[r] & 0xfff);
        order[r] = b;
        sum += tiles_of[b];
    }
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kSortThreads; off <<= 1) {   // inclusive scan of the run sums
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;                               // exclusive
    for (int r = r_begin; r < r_begin + per && r < batch; ++r) {
        prefix[r] = run;
        run += tiles_of[(int)(keys[r] & 0xfff)];
    }
    if (tid == kSortThreads - 1) prefix[batch] = part[tid];
    if (tid == 0) flag[0] = bad;
}

__global__ __launch_bounds__(kItemThreads) void dplan_items_kernel(
    const int32_t* __restrict__ qo, const int32_t* __restrict__ kv, int batch, int num_heads,
    int causal, int block_m, const int32_t* __restrict__ order,
    const int32_t* __restrict__ prefix, int64_t n_items, WorkItem* __restrict__ items) {
    const int64_t i = (int64_t)blockIdx.x * kItemThreads + threadIdx.x;
    if (i >= n_items) return;
    const int x = (int)(i % kDevicePlanXcds);
    const int64_t s = i / kDevicePlanXcds;
    const int hb = num_heads > x ? (num_heads - x + kDevicePlanXcds - 1) / kDevicePlanXcds : 0;
    const int64_t total = prefix[batch];
    WorkItem w{};
    if (s < (int64_t)hb * total) {
        // rank r: prefix[r] * hb <= s < prefix[r + 1] * hb (largest such r)
        int lo = 0, hi = batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)prefix[mid] * hb <= s) lo = mid;
            else hi = mid - 1;
        }
        const int r = lo;
        const int64_t tl = prefix[r + 1] - prefix[r];
        const int64_t rem = s - (int64_t)prefix[r] * hb;
        const int head = x + kDevicePlanXcds * (int)(rem / tl);
        const int t = (int)(tl - 1 - rem % tl);               // heaviest tile first
        const int b = order[r];
        const int qo_len = qo[b + 1] - qo[b];
        const int kv_len = kv[b + 1] - kv[b];
        const int r0 = t * block_m;
        const int rows = qo_len - r0 < block_m ? qo_len - r0 : block_m;
        const int diag0 = causal ? kv_len - qo_len + r0 : kv_len;
        int64_t lim = (int64_t)diag0 + rows;
        lim = lim < 0 ? 0 : (lim > kv_len ? kv_len : lim);
        w.q_row0 = qo[b] + r0;
        w.n_rows = rows;
        w.head0 = head;
        w.n_heads = 1;
        w.kv_start = kv[b];
        w.kv_len = kv_len;
        w.diag0 = diag0;
        w.kv_hi = (int32_t)lim;
    }
    items[i] = w;
}

}  // namespace

int64_t device_plan_max_items(int batch, int64_t max_tq, int num_heads, int block_m) {
    const int64_t heads_per_xcd = (num_heads + kDevicePlanXcds - 1) / kDevicePlanXcds;
    const int64_t tiles = (max_tq + block_m - 1) / block_m + batch;
    return (int64_t)kDevicePlanXcds * heads_per_xcd * tiles;
}

DevicePlanLayout device_plan_layout(int batch, int64_t max_items) {
    auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
    DevicePlanLayout l;
    l.flag = 0;
    l.order = 256;
    l.prefix = l.order + up((int64_t)batch * 4);
    l.items = l.prefix + up((int64_t)(batch + 1) * 4);
    l.bytes = l.items + max_items * (int64_t)sizeof(WorkItem);
    return l;
}

hipError_t device_plan_scratch(void** ptr) {
    // resolved once per device, with that device current
    static std::mutex mu;
    static std::map<int, void*> addr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr.find(dev);
    if (it == addr.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        it = addr.emplace(dev, p).first;
    }
    *ptr = it->second;
    return hipSuccess;
}

hipError_t launch_device_plan(const int32_t* qo, const int32_t* kv, int batch, int64_t max_tq,
                              int64_t max_tk, int num_heads, bool causal, int block_m,
                              void* workspace, int64_t max_items, hipStream_t stream) {
    const DevicePlanLayout l = device_plan_layout(batch, max_items);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* flag = reinterpret_cast<int32_t*>(ws + l.flag);
    int32_t* order = reinterpret_cast<int32_t*>(ws + l.order);
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + l.prefix);
    WorkItem* items = reinterpret_cast<WorkItem*>(ws + l.items);
    hipLaunchKernelGGL(dplan_order_kernel, dim3(1), dim3(kSortThreads), 0, stream, qo, kv, batch,
                       max_tq, max_tk, (int)causal, block_m, flag, order, prefix);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = (max_items + kItemThreads - 1) / kItemThreads;
    hipLaunchKernelGGL(dplan_items_kernel, dim3((unsigned)blocks), dim3(kItemThreads), 0, stream,
                       qo, kv, batch, num_heads, (int)causal, block_m, order, prefix, max_items,
                       items);
    return hipGetLastError();
}

}  // namespace mla
