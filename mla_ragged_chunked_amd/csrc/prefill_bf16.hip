// Ragged MLA prefill attention, bf16 inputs, for gfx950 (CDNA4).
//
// Computes, per work item (one query tile of one sequence, for a block of
// consecutive heads run one after the other), flash-style attention with Dqk = 192 and Dvo = 128: S = sm_scale * Q K^T over the
// visible keys (bottom-right causal or all), online softmax in fp32, O = P V,
// and the natural-log LSE per row. This is the ragged prefill of
// "vllm.v1.attention.backends.mla.prefill.flashinfer" (run() with
// return_lse) at the MLA head dims of "[DeepseekR1] How ragged prefill
// manage kv_cache?" (192 for query/key, 128 for value/output).
//
// Design (MI355X):
//  * One workgroup = 4 waves x 32 query rows (128-row tiles); two workgroups
//    share a CU (2 waves per SIMD, about 230 VGPRs, no AGPRs, 80 KB LDS
//    each), so one wave's VALU work also overlaps the other wave's MFMAs.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//    32 queries (Q stays in VGPRs for the whole head). In the accumulator
//    each lane owns one query column and 16 keys, so row max / row sum are
//    in-lane plus one v_permlane32_swap between the two 32-lane halves.
//  * That accumulator, rounded to bf16, is directly the B operand of
//    O^T = V^T P^T. Accumulator slot (i, half g) of a 32-key block holds key
//    8*(i/4) + 4*g + (i%4), so the V^T A operand for PV MFMA m needs, in
//    k-slot 8*g + e, key 16*m + 8*(e/4) + 4*g + (e%4). V is kept row-major in
//    LDS and read with ds_read_b64_tr_b16 (within each 16-lane group, lane
//    4r+q supplies 4 values of row r and lane j receives column j), each lane
//    addressing the key rows that slot order requires.
//  * K/V tiles of 32 keys are loaded straight from HBM into a 4-stage LDS
//    ring with global_load_lds_dwordx4 (no VGPR staging). K is stored in
//    1 KB blocks of 8 rows x 128 contiguous bytes (8 cache lines per load
//    instruction) with the 16-byte chunks of each row XOR-swizzled so the
//    MFMA fragment reads are bank-conflict free; V rows are 256 B with an XOR
//    swizzle of their chunks for the transposing reads. Addresses are a
//    per-tile scalar base plus a per-lane 32-bit offset computed once per
//    item (recomputed with a clamp only on a sequence's last tile). The ring
//    runs on from one head of the item into the next without draining, and
//    the next head's Q is loaded during the current head's last tile, so the
//    start-up latency is paid once per item rather than once per head. A
//    workgroup may also run two items (two light query tiles of one head,
//    paired by the planner) the same way, the ring streaming from the first
//    into the second.
//  * Software pipeline, one barrier per tile: iteration j publishes tile j+1
//    (and retires tile j-1), puts tile j+3 in flight into tile j-1's stage,
//    runs the softmax of tile j, computes the scores of tile j+1, then PV of
//    tile j, and last the max of tile j+1's scores (with the rare O rescale)
//    while those PV MFMAs run. So after the barrier a wave goes straight from
//    the DMA issue to MFMAs, and every wave always has independent MFMA and
//    VALU work to interleave (softmax first measured slightly faster than
//    scores first; the max at the end of the previous iteration ~6% faster
//    than at the top of its own).
//  * Online softmax in base 2 with sm_scale * log2(e) folded into one FMA.
//    The running max is raised only when a tile's max exceeds it by more
//    than 2^8 (a stale max keeps every p <= 256 and is exact after the final
//    division), so the O rescale is a rarely taken wave-uniform branch (at
//    least once per item, since the max starts at -inf).
//  * Tiles run in three wave-uniform phases: tiles every row of the wave sees
//    in full (no mask code), diagonal / ragged-edge tiles (masked), then
//    tiles only other waves need (loads and barrier only).
//  * The row sum is accumulated from the bf16-rounded p that enter the MFMA
//    (v_dot2 with (1, 1)), so O is normalised by exactly the weights it was
//    built from.
//  * Keys past the sequence end load the last valid row (finite data) and
//    are masked to p = 0; rows with no visible key get O = 0, LSE = -inf.
#include <type_traits>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;                    // 32 query rows per wave
constexpr int kBN = 32;                             // keys per KV tile
constexpr int kKSteps = kDqk / 16;                  // 12
constexpr int kKBytes = kBN * kDqk * 2;             // 12 KB: 12 fragment blocks of 1 KB
constexpr int kVBytes = kBN * kDvo * 2;             // 8 KB: 8 blocks of 4 rows x 256 B
constexpr int kStage = kKBytes + kVBytes;           // 20 KB
constexpr int kStages = 4;
constexpr int kKBlocksPerWave = (kKBytes / 1024) / kWaves;   // 3
constexpr int kVBlocksPerWave = (kVBytes / 1024) / kWaves;   // 2
constexpr int kLoadsPerTile = kKBlocksPerWave + kVBlocksPerWave;
constexpr float kLazyRescale = 8.0f;
// s_waitcnt immediate that waits for vmcnt = 0 only (expcnt and lgkmcnt
// fields at their maxima, gfx9 encoding)
constexpr int kVmcnt0 = (0x7 << 4) | (0xf << 8);
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
// 16-byte chunk slot of chunk c in V row `row` (XOR swizzle over 4-chunk groups)
__device__ __forceinline__ int vslot(int row, int c) { return c ^ ((row & 3) << 2); }

// One 16-byte-per-lane global -> LDS load: lane l's 16 bytes land at
// lds_base + OFF + 16 * l, M0 set by one scalar add (lds_base and sbase are
// wave-uniform values already in SGPRs). Issued as inline asm so the
// compiler does not see LDS DMA in flight (it would wait for all of it
// before every LDS read); the kernel waits for completion itself with
// wait_vmcnt before the barrier that publishes a tile. Nothing else in this
// kernel uses M0.
template <int OFF>
__device__ __forceinline__ void dma16o(const void* sbase, uint32_t voff, uint32_t lds_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_base);
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    // readfirstlane returns int: take each half as uint32_t before widening,
    // or a low word with bit 31 set would sign-extend into the high word
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_add_u32 m0, %0, %1\n\tglobal_load_lds_dwordx4 %2, %3"
                 :: "s"(lds), "n"(OFF), "v"(voff), "s"(base) : "memory", "m0", "scc");
}

// Order of the LDS fragment reads and the MFMAs of one pipelined iteration,
// handed to the scheduler (sched_group_barrier masks: 0x008 MFMA, 0x100 LDS
// read). Left alone it puts each fragment read just before its MFMA, which
// then waits on the LDS. With a next tile: its 12 score MFMAs with the K
// fragments read kKAhead MFMAs ahead, the first V^T reads of PV issued
// during the last score MFMAs, the rest two per PV MFMA. Without one, the 8
// PV MFMAs alone. (Measured on MI355X against the scheduler's own order,
// outputs bit-identical: +1 to +1.6% on the DeepSeek-V3 batch, +1 to +4% on
// long sequences, on three boxes.)
constexpr int kKAhead = 6;
__device__ __forceinline__ void pin_scores_pv_order() {
    __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
    for (int q = 0; q < 12 - kKAhead; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < kKAhead; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < (16 - kKAhead) / 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8 - (16 - kKAhead) / 2, 0);
}
__device__ __forceinline__ void pin_pv_order() {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}
static_assert(kKAhead % 2 == 0 && kKAhead <= 12, "read pattern of pin_scores_pv_order");

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// kPair: two work-list entries per workgroup, each of one head (the paired
// layout of the planner); otherwise one entry of n_heads heads.
template <bool kPaged, bool kPair>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(const WorkItem* __restrict__ items,
                         const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
                         float* __restrict__ lse, int num_heads, float scale_log2, PagedKv pg,
                         const int32_t* __restrict__ block_table) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];

    // This workgroup's items: one, or two run back to back (a second item
    // with n_rows == 0 is absent). A unit is one head of one item; the
    // units run in order (item 0's heads, then item 1's) with the K/V ring
    // streaming from one into the next.
    const WorkItem* wi = items + (int64_t)blockIdx.x * (kPair ? 2 : 1);
    const WorkItem it0 = wi[0];
    if (it0.n_rows <= 0) return;
    const WorkItem it1 = kPair ? wi[1] : it0;
    const int n_it = kPair && it1.n_rows > 0 ? 2 : 1;
    // heads of an item (paired entries hold one head each)
    auto heads_of = [&](const WorkItem& w) { return kPair ? 1 : w.n_heads; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int H = num_heads;
    const int row_w0 = wave * 32;
    const int my_row = row_w0 + l32;
    auto tiles_of = [&](const WorkItem& w) { return (w.kv_hi + kBN - 1) / kBN; };
    const int nt0 = tiles_of(it0);
    const int total_tiles = nt0 * heads_of(it0) + (n_it > 1 ? tiles_of(it1) : 0);

    // Q fragments (B operand): row row_w0 + l32, dims 16*s + 8*g .. +8.
    // Rows past the tile's end load its last row instead (their results are
    // never stored), so every lane loads and no lane needs zero-filling.
    bf16x8_t qf[kKSteps];
    auto load_q = [&](const WorkItem& w, int head) {
        const int q_row = w.q_row0 + (my_row < w.n_rows ? my_row : w.n_rows - 1);
        const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(q + ((int64_t)q_row * H + head) * kDqk);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) qf[s] = src[s * 2 + g];
    };

    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

    // ---- direct global -> LDS staging ----
    // K: 12 blocks of 1 KB per tile; block 3R + G holds rows 8R .. 8R+7, each
    // row's 16-byte chunks 8G .. 8G+7 at slot (chunk ^ (row/2)) % 8.
    // V: 8 blocks of 4 rows x 256 B; row r's chunk c sits at slot vslot(r, c).
    // Keys at or past kv_len load the last valid row instead (finite data;
    // the mask gives those keys p = 0).
    // Per-lane byte offsets (from the tile's first key row) of this wave's
    // loads: 3 K blocks and 2 V blocks; recomputed with the clamp only on a
    // sequence's last tile. The tile's own address is a scalar base.
    const uint32_t krow = (uint32_t)H * kDqk * 2;
    const uint32_t vrow = (uint32_t)H * kDvo * 2;
    // row (key within the tile) and byte column of load j of this lane; the
    // clamped form is only needed on a sequence's last tile, so row and
    // column are recomputed there rather than kept in registers
    auto ld_row = [&](int j) {
        if (j < kKBlocksPerWave) {
            // block bi = 3 R + G: rows 8R .. 8R+7, 16-byte chunks 8G .. 8G+7
            // of each row (128 contiguous bytes per row), chunk order XOR-swizzled
            const int bi = wave * kKBlocksPerWave + j;
            return (bi / 3) * 8 + (lane >> 3);
        }
        return 4 * (wave * kVBlocksPerWave + j - kKBlocksPerWave) + (lane >> 4);
    };
    auto ld_col = [&](int j) {
        const int row = ld_row(j);
        if (j < kKBlocksPerWave)
            return (uint32_t)((((wave * kKBlocksPerWave + j) % 3) * 8 + ((lane & 7) ^ ((row >> 1) & 7))) * 16);
        return (uint32_t)(vslot(row, lane & 15) * 16);
    };
    uint32_t ld_off[kKBlocksPerWave + kVBlocksPerWave];
#pragma unroll
    for (int j = 0; j < kKBlocksPerWave + kVBlocksPerWave; ++j)
        ld_off[j] = (uint32_t)ld_row(j) * (j < kKBlocksPerWave ? krow : vrow) + ld_col(j);
    const uint8_t* k8 = reinterpret_cast<const uint8_t*>(k);
    const uint8_t* v8 = reinterpret_cast<const uint8_t*>(v);

    // ---- issue cursor: the next tile to put in flight ----
    // Contiguous K/V: the cursor's tile addresses advance by one tile of
    // rows per issue and the stage's LDS address rotates through the ring,
    // so an issue costs a few scalar adds (the issue sits between the
    // barrier and the MFMAs). Paged K/V address every tile through its page;
    // the block table is a kernel argument of its own, __restrict__, so its
    // entries are scalar loads (they do not count against the DMA waits),
    // read one issue ahead and clamped only where used.
    const uint32_t smem_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
    const uint32_t wk_lds = (uint32_t)(wave * kKBlocksPerWave * 1024);
    const uint32_t wv_lds = (uint32_t)(kKBytes + wave * kVBlocksPerWave * 1024);
    const uint64_t kstep = (uint64_t)kBN * H * (kDqk * 2);
    const uint64_t vstep = (uint64_t)kBN * H * (kDvo * 2);
    uint32_t iss_lds = smem_lds;
    int iss_g = 0, iss_u = 0, iss_h = 0, iss_kt = 0;
    int iss_nt = 0, iss_nh = 0, iss_head0 = 0, iss_seq = 0, iss_last = -1;
    int64_t iss_row0 = 0;    // row of key 0 of the cursor's item (contiguous K/V)
    const uint8_t* iss_kb = k8;
    const uint8_t* iss_vb = v8;
    // point the cursor at key tile 0 of the first head of item w
    auto iss_enter = [&](const WorkItem& w) {
        iss_nt = tiles_of(w);
        iss_nh = heads_of(w);
        iss_head0 = w.head0;
        iss_seq = w.kv_start;
        iss_last = w.kv_len - 1;
        iss_row0 = kPaged ? 0 : (int64_t)w.kv_start * H;
        iss_kb = k8 + (iss_row0 + iss_head0) * (kDqk * 2);
        iss_vb = v8 + (iss_row0 + iss_head0) * (kDvo * 2);
    };
    // an item without key tiles (its rows see no key) has nothing to load
    iss_enter(it0);
    if (iss_nt == 0 && n_it > 1) {
        iss_u = 1;
        iss_enter(it1);
    }
    auto page_entry = [&](int kt) {
        return block_table[(int64_t)iss_seq * pg.max_pages + (kt * kBN) / pg.page_size];
    };
    int iss_page = 0;
    if constexpr (kPaged) {
        if (total_tiles > 0) iss_page = page_entry(0);
    }
    auto issue_next = [&]() {
        const int key0 = iss_kt * kBN;
        const uint8_t* kb = iss_kb;
        const uint8_t* vb = iss_vb;
        if constexpr (kPaged) {
            const int page = iss_page < 0 ? 0 : (iss_page >= pg.num_pages ? pg.num_pages - 1 : iss_page);
            const uint64_t row0 = (uint64_t)page * pg.page_size + (uint64_t)(key0 % pg.page_size);
            kb = k8 + (row0 * H + iss_head0 + iss_h) * (kDqk * 2);
            vb = v8 + (row0 * H + iss_head0 + iss_h) * (kDvo * 2);
        }
        static_assert(kKBlocksPerWave == 3 && kVBlocksPerWave == 2, "DMA blocks per wave");
        const uint32_t lk = iss_lds + wk_lds, lv = iss_lds + wv_lds;
        auto issue = [&](const uint32_t (&off)[kKBlocksPerWave + kVBlocksPerWave]) __attribute__((always_inline)) {
            dma16o<0>(kb, off[0], lk);
            dma16o<1024>(kb, off[1], lk);
            dma16o<2048>(kb, off[2], lk);
            dma16o<0>(vb, off[3], lv);
            dma16o<1024>(vb, off[4], lv);
        };
        if (key0 + kBN - 1 > iss_last) {
            const int lim = iss_last - key0;
            uint32_t off[kKBlocksPerWave + kVBlocksPerWave];
#pragma unroll
            for (int j = 0; j < kKBlocksPerWave + kVBlocksPerWave; ++j) {
                const int r = ld_row(j) < lim ? ld_row(j) : lim;
                off[j] = (uint32_t)r * (j < kKBlocksPerWave ? krow : vrow) + ld_col(j);
            }
            issue(off);
        } else {
            issue(ld_off);
        }
        ++iss_g;
        iss_lds = iss_lds + kStage == smem_lds + kStages * kStage ? smem_lds : iss_lds + kStage;
        if (++iss_kt == iss_nt) {
            iss_kt = 0;
            if (++iss_h == iss_nh) {
                // the next item (the cursor only gets here while tiles remain,
                // so that item has key tiles)
                iss_h = 0;
                if (++iss_u < n_it) iss_enter(it1);
            } else {
                iss_kb = k8 + (iss_row0 + iss_head0 + iss_h) * (kDqk * 2);
                iss_vb = v8 + (iss_row0 + iss_head0 + iss_h) * (kDvo * 2);
            }
        } else if constexpr (!kPaged) {
            iss_kb += kstep;
            iss_vb += vstep;
        }
        if constexpr (kPaged) {
            if (iss_g < total_tiles) iss_page = page_entry(iss_kt);
        }
    };

    // LDS offsets of this lane's K fragment (row l32, chunk 2s + g) for
    // k-steps s = 4u + t: block 3 (l32/8) + u, slot 8 (l32%8) + ((2t+g) ^ ((l32/2)%8))
    int k_off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        k_off[t] = (l32 >> 3) * 3 * 1024 + ((l32 & 7) * 8 + ((2 * t + g) ^ ((l32 >> 1) & 7))) * 16;

    // ---- compute pieces ----
    int my_lim = 0;    // keys visible to this lane's row in the current item
    auto scores = [&](int kt, int stage, auto masked, f32x16_t& sacc) {
        constexpr bool kMasked = decltype(masked)::value;
        const uint8_t* ks = smem + stage * kStage;
        sacc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ks + k_off[s & 3] + (s >> 2) * 1024);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
        }
        if constexpr (kMasked) {
            // slot i holds key kt * kBN + (i/4) * 8 + 4 g + i%4: it is visible
            // iff its offset (i/4) * 8 + i%4 inside the tile is below lim_rel,
            // so each compare takes an inline constant and no per-slot key
            // has to stay in a register
            const int lim_rel = my_lim - kt * kBN - g * 4;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sacc[i] = (i >> 2) * 8 + (i & 3) < lim_rel ? sacc[i] : -INFINITY;
        }
    };
    auto tile_max = [&](const f32x16_t& sv) {
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
        return xor32_max(mx) * scale_log2;
    };
    // V^T fragment for dv block db, key step mm (16 keys): two transposing
    // reads of 4 keys each. Lane (g, h = bit 4, j = low 4 bits, r = j/4,
    // q = j%4) supplies row mm*16 + t*8 + g*4 + r, dims db*32 + h*16 + 4q.
    // The swizzle only depends on row % 4 = r, so the per-lane offset of
    // (db, mm = 0, t = 0) is computed once and (mm, t) become immediates.
    int v_off[4];
    {
        const int tr_h = (lane >> 4) & 1;
        const int tr_r = (lane & 15) >> 2;
        const int tr_q = lane & 3;
        const int row = g * 4 + tr_r;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int chunk = db * 4 + tr_h * 2 + (tr_q >> 1);
            v_off[db] = kKBytes + row * 256 + vslot(row, chunk) * 16 + (tr_q & 1) * 8;
        }
    }
    auto vfrag = [&](const uint8_t* st, int db, int mm) {
        bf16x8_t a;
        const uint8_t* base = st + v_off[db];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t* p = base + (mm * 16 + t * 8) * 256;
            const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
            const bf16x4_t y = __builtin_bit_cast(bf16x4_t, x);
            a[t * 4 + 0] = y[0];
            a[t * 4 + 1] = y[1];
            a[t * 4 + 2] = y[2];
            a[t * 4 + 3] = y[3];
        }
        return a;
    };
    auto softmax = [&](const f32x16_t& sacc, bf16x8_t (&pf)[2]) {
        const float msub = m_run == -INFINITY ? 0.0f : m_run;
        float lsum = l_run;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            bf16x8_t frag;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mm * 8 + e], scale_log2, -msub));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mm * 8 + e + 1], scale_log2, -msub));
                const bf16x2_t pk = {(__bf16)p0, (__bf16)p1};
                frag[e] = pk[0];
                frag[e + 1] = pk[1];
                lsum = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes, lsum, false);
            }
            pf[mm] = frag;
        }
        l_run = lsum;
    };
    auto pv = [&](int stage, const bf16x8_t (&pf)[2]) {
        const uint8_t* st = smem + stage * kStage;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                const bf16x8_t a = vfrag(st, db, mm);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[mm], oacc[db], 0, 0, 0);
            }
        }
    };

    // O = acc / l and LSE = (m + log2 l) ln 2 for one head of item w
    // (waves with rows in it)
    auto store_out = [&](const WorkItem& w, int head) {
        if (w.n_rows - row_w0 <= 0) return;
        const float ltot = xor32_sum(l_run);
        if (my_row >= w.n_rows) return;
        const float inv = ltot > 0.f ? 1.0f / ltot : 0.0f;
        const int64_t orow = (int64_t)(w.q_row0 + my_row) * H + head;
        uint16_t* dst = out + orow * kDvo;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int dv = db * 32 + grp * 8 + g * 4;
                bf16x4_t o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][grp * 4 + e] * inv);
                *reinterpret_cast<bf16x4_t*>(dst + dv) = o4;
            }
        }
        if (g == 0 && lse != nullptr)
            lse[orow] = ltot > 0.f ? (m_run + __log2f(ltot)) * kLn2 : -INFINITY;
    };

    // Software pipeline over the global tile index gt (all units' tiles in
    // order; tile gt lives in stage gt % kStages): the iteration for tile
    // gt publishes tile gt+1 (one barrier, which also retires tile gt-1),
    // puts tile gt+3 in flight into tile gt-1's stage, computes the scores
    // of the unit's next tile and runs softmax + PV of tile gt.
    auto sync_top = [&](int gt) {
        // loads issued so far: tiles 0 .. gt+2; tile gt+1 must be complete
        if (gt + 2 < total_tiles) wait_vmcnt<kLoadsPerTile>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (gt + 3 < total_tiles) issue_next();
    };

    // A wave whose rows see no key of the first unit does not read its Q
    // (it loads the Q of its first unit with work when it gets there).
    auto wave_hi_of = [&](const WorkItem& w) {
        int wr = w.n_rows - row_w0;
        wr = wr < 0 ? 0 : (wr > 32 ? 32 : wr);
        return wr > 0 ? lim_of(row_w0 + wr - 1, w.diag0, w.kv_len) : 0;
    };
    bool q_ready = wave_hi_of(it0) > 0;     // qf holds the Q of the next unit with work
    if (q_ready) load_q(it0, it0.head0);
    for (int t = 0; t < 3 && t < total_tiles; ++t) issue_next();
    // Q and tile 0 must be complete: tiles 1 and 2 may still be in flight
    if (total_tiles > 2) wait_vmcnt<2 * kLoadsPerTile>();
    else if (total_tiles > 1) wait_vmcnt<kLoadsPerTile>();
    else wait_vmcnt<0>();
    __syncthreads();

    int gbase = 0;
    for (int u = 0; u < n_it; ++u) {
        const WorkItem w = u == 0 ? it0 : it1;
        const int n_tiles = tiles_of(w);
        int wave_rows = w.n_rows - row_w0;
        wave_rows = wave_rows < 0 ? 0 : (wave_rows > 32 ? 32 : wave_rows);
        const int wave_lo = wave_rows > 0 ? lim_of(row_w0, w.diag0, w.kv_len) : 0;
        const int wave_hi = wave_rows > 0 ? lim_of(row_w0 + wave_rows - 1, w.diag0, w.kv_len) : 0;
        my_lim = lim_of(my_row, w.diag0, w.kv_len);
        const int n_full = __builtin_amdgcn_readfirstlane(wave_lo / kBN);
        const int n_wave = __builtin_amdgcn_readfirstlane((wave_hi + kBN - 1) / kBN);
        for (int h = 0; h < heads_of(w); ++h, gbase += n_tiles) {
            // the unit after this one, if any, and whether this wave has work there
            const bool next_same = h + 1 < heads_of(w);
            const bool has_next = next_same || u + 1 < n_it;
            const WorkItem wn = next_same || u + 1 >= n_it ? w : it1;
            const int head_next = next_same ? w.head0 + h + 1 : wn.head0;
            const bool next_work = has_next && (next_same ? n_wave > 0 : wave_hi_of(wn) > 0);
            int j = 0;
            bool loaded_next = false;
            if (n_wave > 0) {
                if (!q_ready) {
                    // no Q was loaded for this unit: load it and wait (this
                    // also waits for the ring's loads in flight)
                    load_q(w, w.head0 + h);
                    __builtin_amdgcn_s_waitcnt(kVmcnt0);
#pragma unroll
                    for (int s = 0; s < kKSteps; ++s) asm volatile("" : "+v"(qf[s]));
                }
#pragma unroll
                for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
                m_run = -INFINITY;
                l_run = 0.f;
                // The running max for a tile is raised (lazily) before its
                // softmax: the iteration that computes a tile's scores does
                // it after its own PV MFMAs are issued, so the max's
                // dependent VALU chain overlaps them instead of sitting
                // between the next barrier and the next MFMAs (the O rescale
                // still follows that PV, the order of the arithmetic is
                // unchanged).
                auto update_max = [&](const f32x16_t& sv) {
                    const float mt = tile_max(sv);
                    if (__builtin_expect(__any(mt > m_run + kLazyRescale), 0)) {
                        const float m_new = fmaxf(m_run, mt);
                        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                        m_run = m_new;
                        l_run *= alpha;
#pragma unroll
                        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
                    }
                };
                // One pipelined iteration: consumes the scores of tile j in
                // s_cur and, unless kNext == 0, leaves those of tile j + 1 in
                // s_nxt (kNext: 0 = no next tile, 1 = unmasked, 2 = masked).
                // The loops below alternate two score buffers, so nothing is
                // copied.
                auto iteration = [&](int jj, auto next_kind, const f32x16_t& s_cur, f32x16_t& s_nxt) {
                    constexpr int kNext = decltype(next_kind)::value;
                    const int gt = gbase + jj;
                    sync_top(gt);
                    if constexpr (kNext == 0) {
                        // The next unit's Q: issued after this tile's DMA, so
                        // waiting for it later never waits on a younger tile.
                        if (next_work) {
                            load_q(wn, head_next);
                            loaded_next = true;
                        }
                    }
                    bf16x8_t pf[2];
                    softmax(s_cur, pf);
                    if constexpr (kNext == 1) scores(jj + 1, (gt + 1) % kStages, std::false_type{}, s_nxt);
                    if constexpr (kNext == 2) scores(jj + 1, (gt + 1) % kStages, std::true_type{}, s_nxt);
                    pv(gt % kStages, pf);
                    if constexpr (kNext != 0) pin_scores_pv_order();
                    else pin_pv_order();
                    if constexpr (kNext != 0) update_max(s_nxt);
                };
                // The first tile always takes the masked form (a no-op on a
                // fully visible tile): one straight-line path into the loops,
                // on which the compiler sees the Q wait.
                f32x16_t sa, sb;
                scores(0, gbase % kStages, std::true_type{}, sa);
                update_max(sa);
                // tiles j with an unmasked successor, then with a masked one
                for (; j + 2 < n_full; j += 2) {
                    iteration(j, std::integral_constant<int, 1>{}, sa, sb);
                    iteration(j + 1, std::integral_constant<int, 1>{}, sb, sa);
                }
                if (j + 1 < n_full) {
                    iteration(j, std::integral_constant<int, 1>{}, sa, sb);
                    sa = sb;
                    ++j;
                }
                for (; j + 2 < n_wave; j += 2) {
                    iteration(j, std::integral_constant<int, 2>{}, sa, sb);
                    iteration(j + 1, std::integral_constant<int, 2>{}, sb, sa);
                }
                if (j + 1 < n_wave) {
                    iteration(j, std::integral_constant<int, 2>{}, sa, sb);
                    sa = sb;
                    ++j;
                }
                iteration(j, std::integral_constant<int, 0>{}, sa, sb);
                ++j;
                // The next unit's Q loads are the youngest vector-memory
                // reads: completing them here costs no ring tile. The empty
                // asm then redefines the Q registers, so the compiler no
                // longer sees loads in flight into them and puts no waits of
                // its own in the loops.
                if (loaded_next) {
                    __builtin_amdgcn_s_waitcnt(kVmcnt0);
#pragma unroll
                    for (int s = 0; s < kKSteps; ++s) asm volatile("" : "+v"(qf[s]));
                }
            } else {
                // no row of this wave sees a key of this unit: O = 0, LSE = -inf
#pragma unroll
                for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
                m_run = -INFINITY;
                l_run = 0.f;
            }
            store_out(w, w.head0 + h);
            q_ready = loaded_next;
            // tiles only other waves need: barriers and loads
            for (; j < n_tiles; ++j) sync_top(gbase + j);
        }
    }
    wait_vmcnt<0>();
}

}  // namespace

int prefill_bf16_block_m() { return kBM; }

hipError_t launch_prefill_bf16(const WorkItem* items, int64_t n_items, const void* q,
                               const void* k, const void* v, void* out, float* lse,
                               int num_heads, float sm_scale, hipStream_t stream,
                               const PagedKv* paged, int items_per_wg) {
    if (n_items <= 0) return hipSuccess;
    if (items_per_wg < 1 || items_per_wg > 2 || n_items % items_per_wg != 0)
        return hipErrorInvalidValue;
    const int64_t blocks = n_items / items_per_wg;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    const PagedKv pg = paged != nullptr ? *paged : PagedKv{nullptr, 0, 0, 0};
    const int32_t* table = paged != nullptr ? pg.block_table : nullptr;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, items,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse,
                           num_heads, scale_log2, pg, table);
    };
    if (paged != nullptr)
        items_per_wg == 2 ? launch(prefill_bf16_kernel<true, true>)
                          : launch(prefill_bf16_kernel<true, false>);
    else
        items_per_wg == 2 ? launch(prefill_bf16_kernel<false, true>)
                          : launch(prefill_bf16_kernel<false, false>);
    return hipGetLastError();
}

}  // namespace mla
