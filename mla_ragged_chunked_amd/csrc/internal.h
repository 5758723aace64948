// Internal declarations shared by the C ABI, the planner and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

namespace mla {

constexpr int kDqk = 192;
constexpr int kDvo = 128;
constexpr int kDlat = 512;
constexpr int kDrope = 64;
constexpr int kDnope = 128;

// One work item = one query tile of one sequence for a block of heads
// [head0, head0 + n_heads), processed one head after the other. 32 bytes.
//   row r of the tile (0 <= r < n_rows) sees keys [0, lim(r)) of its sequence,
//   lim(r) = min(kv_len, max(0, diag0 + r + 1)).
// Non-causal tiles carry diag0 = kv_len, so lim(r) = kv_len.
struct WorkItem {
    int32_t q_row0;    // global token index of the tile's first query row
    int32_t n_rows;    // rows in the tile; 0 = padding item (kernel returns)
    int32_t head0;     // first head of the block
    int32_t n_heads;   // heads in the block (>= 1 for a real item)
    int32_t kv_start;  // global token index of the sequence's first key
    int32_t kv_len;
    int32_t diag0;
    int32_t kv_hi;     // lim(n_rows - 1): keys the tile must visit (per head)
};
static_assert(sizeof(WorkItem) == 32, "work item layout");

// Paged K/V source. The caches are [num_pages, page_size, H, D]; key j of
// sequence b sits in page block_table[b * max_pages + j / page_size], slot
// j % page_size. page_size is a multiple of 32, so a 32-key tile lies in one
// page. In paged mode WorkItem::kv_start holds the sequence index b. Page
// indices read from the (device) table are clamped to [0, num_pages).
struct PagedKv {
    const int32_t* block_table;  // device int32 [batch, max_pages]
    int32_t max_pages;
    int32_t page_size;
    int32_t num_pages;
};

// One work item of the weight-absorbed (latent-cache) prefill: a tile of
// consecutive flat query rows of one sequence, flat row rho = token * H +
// head, over the keys [kv_lo, kv_hi) of that sequence. Row rho sees keys
// [0, lim(rho)) of its sequence,
//   lim(rho) = min(kv_len, max(0, diag_base + (rho - seq_row0) / H + 1)),
// diag_base = kv_len - qo_len when causal, kv_len otherwise. When the keys of
// a tile are split over several items (KV splits), each writes a partial
// (O, LSE) over its keys into split slot `part` and a merge combines them.
// 48 bytes.
struct LatentItem {
    int32_t row0;       // first flat row of the tile
    int32_t n_rows;     // rows in the tile; 0 = padding item (kernel returns)
    int32_t seq_row0;   // flat row of the sequence's first token, head 0
    int32_t kv_hi;      // end of the item's keys (at most lim of the tile's last row)
    int32_t kv_start;   // global token index of the sequence's first key
    int32_t kv_len;
    int32_t diag_base;
    int32_t kv_lo;      // first key of the item, a multiple of 32
    int32_t part;       // -1: final output; else the KV split slot of the partial
    int32_t pad[3];
};
static_assert(sizeof(LatentItem) == 48, "latent work item layout");

// Query-tile heights of the two prefill kernels (each kernel file owns its
// tile shape; the planner asks for it).
int prefill_bf16_block_m();
int prefill_fp32_block_m();

// Build the ordered work list (host only). Returns false with `err` set on
// invalid input. `block_m` is the query-tile height, `n_xcd` the number of
// XCDs work is grouped for (1 = no grouping).
// `heads_per_item` is the head-block size (it must divide num_heads); 0
// means automatic (one head per item).
// `kv_start_is_seq` stores the sequence index in kv_start (paged K/V).
// bf16 prefill: two neighbouring light tiles of a sequence share one
// workgroup while the keys they see add up to at most this many (measured on
// MI355X against one tile per workgroup: +7% on 64 sequences of 512 tokens
// and 32 of 1024, +6% on 16 of 2048, +3% on 8 of 4096, +1% on the
// DeepSeek-V3 batch; long, skewed and non-causal batches unchanged; caps
// from 384 to 768 keys measured the same). The same switch also pairs the
// equal tiles of non-causal sequences (planner.cpp, step 6).
constexpr int kPrefillPairMaxKeys = 512;
// `pair_max_keys` > 0 may pair tiles (see planner.cpp); `items_per_wg`, if
// not NULL, receives the entries per workgroup slot of the list: 2 when a
// pair formed (a second entry with n_rows == 0 is absent), else 1.
bool build_work_list(const int32_t* qo_indptr, const int32_t* kv_indptr, int batch,
                     int num_heads, bool causal, int block_m, int n_xcd, int heads_per_item,
                     std::vector<WorkItem>& out, std::string& err, bool kv_start_is_seq = false,
                     int pair_max_keys = 0, int* items_per_wg = nullptr);

// Work list of the weight-absorbed prefill (host only): tiles of `block_m`
// flat rows, grouped and ordered for the XCDs like build_work_list.
// `kv_start_is_seq` stores the sequence index in kv_start (paged cache).
// `splits` >= 1: the keys of every tile are cut into that many item ranges
// of whole 32-key tiles (1 = no split, items write the final output).
bool build_latent_work_list(const int32_t* qo_indptr, const int32_t* kv_indptr, int batch,
                            int num_heads, bool causal, int block_m, int n_xcd,
                            std::vector<LatentItem>& out, std::string& err,
                            bool kv_start_is_seq = false, int splits = 1);
// KV splits chosen for a call: more than one only when the row tiles alone
// cannot fill the chip and the keys are long enough to share out.
int latent_kv_splits(const int32_t* qo_indptr, const int32_t* kv_indptr, int batch,
                     int num_heads, bool causal, int block_m);
int prefill_absorbed_block_m();

// Device-side partitioner (device_plan.hip). The workspace holds, at these
// byte offsets: a flag word (nonzero = some sequence had invalid indptrs and
// was skipped), the sequence order, the tile prefix sums and the work list.
constexpr int kDevicePlanMaxBatch = 4096;
constexpr int kDevicePlanXcds = 8;
struct DevicePlanLayout {
    int64_t flag, order, prefix, items, bytes;
};
// Size of the device-plan workspace held in a file-scope device array for
// the allocation-free entry point (it fits, e.g., 128 heads over 262,144
// query tokens in 64 sequences: 7.9 MB of work list).
constexpr int64_t kDevicePlanScratchBytes = INT64_C(16) << 20;
// Device address of that array on the current device (resolved with
// hipGetSymbolAddress on the first call per device).
hipError_t device_plan_scratch(void** ptr);
int64_t device_plan_max_items(int batch, int64_t max_tq, int num_heads, int block_m);
DevicePlanLayout device_plan_layout(int batch, int64_t max_items);
hipError_t launch_device_plan(const int32_t* qo_indptr, const int32_t* kv_indptr, int batch,
                              int64_t max_tq, int64_t max_tk, int num_heads, bool causal,
                              int block_m, void* workspace, int64_t max_items, hipStream_t stream);

// Kernel launchers (one kernel each, enqueued on `stream`).
// `paged` == nullptr: contiguous K/V ([Tk, H, D], rows from kv_start).
// `items_per_wg` (1 or 2, bf16 only): work-list entries per workgroup.
hipError_t launch_prefill_bf16(const WorkItem* items, int64_t n_items, const void* q,
                               const void* k, const void* v, void* out, float* lse,
                               int num_heads, float sm_scale, hipStream_t stream,
                               const PagedKv* paged = nullptr, int items_per_wg = 1);
hipError_t launch_prefill_fp32(const WorkItem* items, int64_t n_items, const void* q,
                               const void* k, const void* v, void* out, float* lse,
                               int num_heads, float sm_scale, hipStream_t stream,
                               const PagedKv* paged = nullptr);
// `paged` == nullptr: contiguous cache [Tk, 576] (rows from kv_start); else
// a page pool [num_pages, page_size, 576] (PagedKv with H = 1).
// Items with part >= 0 write partial states: O (bf16, normalised) to
// part_o[(part * part_rows + rho) * 512], LSE (fp32) to
// part_lse[part * part_rows + rho].
hipError_t launch_prefill_absorbed(const LatentItem* items, int64_t n_items, const void* q,
                                   const void* kv, void* out, float* lse, int num_heads,
                                   float sm_scale, hipStream_t stream,
                                   const PagedKv* paged = nullptr, uint16_t* part_o = nullptr,
                                   float* part_lse = nullptr, int64_t part_rows = 0);
// Combine `splits` partial states per row into out (bf16 [rows, 512]) and lse
// (fp32 [rows], may be NULL).
hipError_t launch_merge_splits(const uint16_t* part_o, const float* part_lse, int splits,
                               int64_t rows, void* out, float* lse, hipStream_t stream);
hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b,
                        const float* lse_b, void* o, float* lse, int64_t num_rows,
                        int dtype_bf16, hipStream_t stream);
// Decompression fused into the prefill: `tiles` are query tiles of
// decompress_prefill_block_m() rows (one head each, head fields unused)
// sorted by kv_hi, heaviest first; the first n_busy have kv_hi > 0.
int decompress_prefill_block_m();
hipError_t launch_decompress_prefill(const WorkItem* tiles, int64_t n_tiles, int64_t n_busy,
                                     const void* q, const void* c_kv, const void* k_rope,
                                     const void* w_uk, const void* w_uv, void* out, float* lse,
                                     int num_heads, float sm_scale, hipStream_t stream);
hipError_t launch_decompress(const void* c_kv, const void* k_rope, const void* w_uk,
                             const void* w_uv, int64_t num_tokens, int num_heads,
                             void* k_out, void* v_out, hipStream_t stream);

}  // namespace mla
