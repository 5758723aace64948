// Weight-absorbed MLA prefill over the latent cache, bf16, for gfx950.
//
// The absorbed path ("[DeepseekR1] How ragged prefill manage kv_cache?",
// sglang issue 3849: forward_absorb, which attends the compressed cache
// directly instead of decompressing it) is multi-query attention: every head
// h of query token t has a 576-dim absorbed query q[t,h] (latent 512 + RoPE
// 64), every key token j one shared 576-dim cache row kv[j] = [c_kv | k_rope],
// and the value of key j is the first 512 dims of that same row. The output
// O[t,h] (512 dims, still in the latent space) and the natural-log LSE per
// (t, h) follow the same visible-key rule (bottom-right causal or all) and
// scaling as the MHA prefill.
//
// Design (MI355X):
//  * Query rows are the flat (token, head) pairs, token-major: row rho is
//    q[rho / H, rho % H], contiguous in memory, and sees the keys of token
//    rho / H. One workgroup = 128 consecutive rows of one sequence, 4 waves x
//    32 rows, one wave per SIMD: Q (144 VGPRs) stays in registers, the 512-dim
//    O of 32 rows (256 fp32 per lane) lives in AGPRs.
//  * Each 32-key tile (36 KB: 36 blocks of 8 keys x 64 dims, chunk-swizzled)
//    is loaded straight into LDS with global_load_lds_dwordx4 and serves both
//    products: its fragments are the A operand of S^T = K Q^T
//    (v_mfma_f32_32x32x16_bf16, 36 k-steps in one accumulator chain: dependent
//    MFMAs issue back to back), and transposing reads (ds_read_b64_tr_b16) of
//    its first 512 dims are the V^T operand of O^T = V^T P^T (16 dv blocks x
//    2 k-steps). LDS fragments are read three MFMAs ahead of use.
//  * Each wave reads the whole tile (36 KB as 16-byte rows, 32 KB through
//    transposing reads) for its 32 rows; the chunk swizzle keeps both read
//    kinds free of bank conflicts on the 64-bank LDS. One wave per SIMD
//    issues all of its MFMAs, LDS reads and softmax in order, which is what
//    bounds the kernel (not the LDS bandwidth nor the matrix cores).
//  * Iteration j computes the scores, softmax and PV of tile j, so a tile's
//    stage is free again at the next barrier: the 4-stage ring (144 KB) keeps
//    tiles j+1 .. j+3 in flight.
//  * Online softmax in base 2, lazy rescale (threshold 2^8) and the row sum
//    from the bf16-rounded p, as in the MHA kernel. The rare O rescale runs in
//    place on the AGPRs.
//  * Keys past the sequence end load the last valid row (finite data) and are
//    masked to p = 0; rows with no visible key get O = 0, LSE = -inf.
#include <type_traits>

#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kDk = kDlat + kDrope;                 // 576
constexpr int kDv = kDlat;                          // 512
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;                    // 128 rows per tile
constexpr int kBN = 32;                             // keys per KV tile
constexpr int kKSteps = kDk / 16;                   // 36
constexpr int kGroups = kDk / 64;                   // 9 groups of 64 dims per key row
constexpr int kTileBytes = kBN * kDk * 2;           // 36 KB
constexpr int kStages = 4;
constexpr int kLoadsPerTile = kGroups;              // each wave: its 8 keys x 9 groups
constexpr int kDvBlocks = kDv / 32;                 // 16
constexpr float kLazyRescale = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(kWaves * 8 == kBN, "one 8-key row group per wave");

__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Chunk swizzle of tile row (key) `row`: the 16-byte chunk c of a row sits
// at slot c ^ swz(row). 128-byte rows, so two rows share one 256-byte bank
// period. A 16-byte read by 16 lanes (keys of one parity, same chunk) needs
// swz to be a permutation over those 8 keys; a transposing read by 32 lanes
// (keys 4i..4i+3, four chunks of one aligned group) needs keys 4i and 4i+2 in
// different 4-slot halves, hence bit 2 of swz from bit 1 of the key.
__device__ __forceinline__ int swz(int row) {
    return ((row >> 1) & 1) << 2 | ((row >> 2) & 1) << 1 | ((row >> 3) & 1);
}

// One 16-byte-per-lane global -> LDS load (lane l's 16 bytes land at
// lds_dst + 16 l), issued as inline asm so the compiler does not wait for it
// before LDS reads; completion is awaited with wait_vmcnt before the barrier
// that publishes a tile. Nothing else in this kernel uses M0.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, const void* lds_dst) {
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    // each half as uint32_t before widening: readfirstlane returns int
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(voff), "s"(base) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// x *= alpha on an accumulator held in an AGPR, in place. The leading s_nops
// cover the wait states after an MFMA that wrote x, the trailing one those
// before an MFMA that reads it.
__device__ __forceinline__ void agpr_scale(float& x, float alpha) {
    float t;
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                 "v_accvgpr_read_b32 %1, %0\n\t"
                 "v_mul_f32 %1, %1, %2\n\t"
                 "v_accvgpr_write_b32 %0, %1\n\t"
                 "s_nop 7"
                 : "+a"(x), "=&v"(t)
                 : "v"(alpha));
}

// kPaged: the cache is a page pool [num_pages, page_size, 576] read through
// a block table, and LatentItem::kv_start holds the sequence index.
template <bool kPaged>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_absorbed_kernel(const LatentItem* __restrict__ items, const uint16_t* __restrict__ q,
                             const uint16_t* __restrict__ kv, uint16_t* __restrict__ out,
                             float* __restrict__ lse, int num_heads, float scale_log2, PagedKv pg,
                             const int32_t* __restrict__ block_table, uint16_t* __restrict__ part_o,
                             float* __restrict__ part_lse, int64_t part_rows) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kTileBytes];

    const LatentItem it = items[blockIdx.x];
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
    // keys visible to flat row rho: those of its token, rho's token index in
    // the sequence being (rho - seq_row0) / H
    auto lim_of_row = [&](int r) __attribute__((always_inline)) {
        const int tok = (it.row0 + r - it.seq_row0) / H;
        int n = it.diag_base + tok + 1;
        n = n < 0 ? 0 : n;
        return n > it.kv_len ? it.kv_len : n;
    };
    const int wave_lo = wave_rows > 0 ? lim_of_row(row_w0) : 0;
    const int wave_hi = wave_rows > 0 ? lim_of_row(row_w0 + wave_rows - 1) : 0;
    const int my_row = row_w0 + l32;
    const int my_lim = lim_of_row(my_row < it.n_rows ? my_row : it.n_rows - 1);

    // Q fragments (B operand): this lane's row, dims 16 s + 8 g .. +8; rows
    // past the tile's end load its last row (their results are never stored).
    // Plain loads, issued after the first K/V tiles and completed by a wait
    // before the key loop; the registers then pass through an empty asm
    // (below), without which the compiler kept counting the loads as in
    // flight and waited for them before the score MFMAs of every tile
    // (waits that also drained the ring's tiles in flight).
    bf16x8_t qf[kKSteps];
    const bf16x8_t* q_src;
    {
        const int64_t rho = (int64_t)it.row0 + (my_row < it.n_rows ? my_row : it.n_rows - 1);
        q_src = reinterpret_cast<const bf16x8_t*>(q + rho * kDk) + g;
    }

    f32x16_t oacc[kDvBlocks];
#pragma unroll
    for (int db = 0; db < kDvBlocks; ++db) oacc[db] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

    // ---- direct global -> LDS staging ----
    // Block 9 R + G (1 KB) holds keys 8R .. 8R+7, dims 64 G .. 64 G + 63:
    // key row r at 128 r, its 16-byte chunk c (of the group) at slot
    // c ^ swz(key). Wave w loads keys 8w .. 8w+7 of all nine groups.
    const uint32_t krow = (uint32_t)kDk * 2;            // one shared cache row
    const int last_key = it.kv_len - 1;
    const int ld_row = 8 * wave + (lane >> 3);
    uint32_t ld_col[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) ld_col[j] = (uint32_t)(8 * j + ((lane & 7) ^ swz(ld_row))) * 16;
    const uint8_t* kvseq = reinterpret_cast<const uint8_t*>(kv + (kPaged ? 0 : (int64_t)it.kv_start * kDk));
    // Table entry of key tile kt (paged cache). The block table is a kernel
    // argument of its own, __restrict__, so this is a scalar load, which does
    // not count against the DMA waits; the raw value is clamped into the pool
    // only where it is used, one issue later, so its latency is not waited for.
    auto page_entry = [&](int kt) __attribute__((always_inline)) {
        return block_table[(int64_t)it.kv_start * pg.max_pages + (it.kv_lo + kt * kBN) / pg.page_size];
    };
    // tile kt into `stage` (`entry`: its table entry, paged cache only)
    auto issue_tile = [&](int kt, int stage, int entry) __attribute__((always_inline)) {
        uint8_t* dst = smem + stage * kTileBytes + wave * kGroups * 1024;
        const int key0 = it.kv_lo + kt * kBN;
        uint64_t row0 = (uint64_t)key0;
        if constexpr (kPaged) {
            const int page = entry < 0 ? 0 : (entry >= pg.num_pages ? pg.num_pages - 1 : entry);
            row0 = (uint64_t)page * pg.page_size + (uint64_t)(key0 % pg.page_size);
        }
        const uint8_t* src = kvseq + row0 * krow;
        int r = ld_row;
        if (key0 + kBN - 1 > last_key) r = r < last_key - key0 ? r : last_key - key0;
        const uint32_t roff = (uint32_t)r * krow;
#pragma unroll
        for (int j = 0; j < kGroups; ++j) dma16(src, roff + ld_col[j], dst + j * 1024);
    };

    // LDS offsets of this lane's K fragment (key l32, chunk 2s + g) for
    // k-steps s = 4u + t: block 9 (l32/8) + u, row l32 % 8, slot (2t+g) ^ swz(l32)
    int k_off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        k_off[t] = 9 * (l32 >> 3) * 1024 + (l32 & 7) * 128 + (((2 * t + g) ^ swz(l32)) & 7) * 16;
    // V^T fragment (dv block db, key step mm): two transposing reads. Lane
    // (g, h = bit 4, r = bits 2-3, q = bits 0-1) supplies key
    // 16 mm + 8 t + 4 g + r, dims 32 db + 16 h + 4 q .. +4: chunk
    // 4 db + 2 h + q/2 = group db/2, chunk-in-group 4 (db&1) + 2 h + q/2.
    // The swizzle depends on (db & 1, t) only, so the offset for those four
    // combinations is per lane and (mm, t, db/2) become immediates.
    int v_off[2][2];
    {
        const int tr_h = (lane >> 4) & 1;
        const int tr_r = (lane & 15) >> 2;
        const int tr_q = lane & 3;
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int key = 8 * t + 4 * g + tr_r;            // + 16 mm: same swizzle
                const int c8 = 4 * odd + 2 * tr_h + (tr_q >> 1);
                v_off[odd][t] = (key & 7) * 128 + ((c8 ^ swz(key)) & 7) * 16 + (tr_q & 1) * 8;
            }
        }
    }

    // ---- compute pieces ----
    // LDS fragments are read kPre MFMAs ahead of their use: with one wave
    // per SIMD nothing else hides the LDS latency. (Measured on MI355X once
    // the ring stayed in flight: 3 ahead ~0.6% faster than 4 on prefill,
    // decode unchanged; 6 ahead 8% slower.)
    constexpr int kPre = 3;
    auto kfrag = [&](const uint8_t* ks, int s) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8_t*>(ks + k_off[s & 3] + (s >> 2) * 1024);
    };
    // S^T of tile kt: one accumulator chain over the 36 k-steps
    auto scores = [&](int kt, int stage, auto masked, f32x16_t& sacc) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked)::value;
        const uint8_t* ks = smem + stage * kTileBytes;
        bf16x8_t a[kPre];
#pragma unroll
        for (int s = 0; s < kPre; ++s) a[s] = kfrag(ks, s);
        f32x16_t acc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % kPre], qf[s], acc, 0, 0, 0);
            if (s + kPre < kKSteps) a[s % kPre] = kfrag(ks, s + kPre);
        }
        sacc = acc;
        if constexpr (kMasked) {
            const int key0 = it.kv_lo + kt * kBN;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + (i >> 2) * 8 + g * 4 + (i & 3);
                sacc[i] = key < my_lim ? sacc[i] : -INFINITY;
            }
        }
    };
    auto vfrag = [&](const uint8_t* st, int i) __attribute__((always_inline)) {
        const int db = i >> 1, mm = i & 1;
        bf16x8_t a;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t* p = st + v_off[db & 1][t] + (9 * (2 * mm + t) + (db >> 1)) * 1024;
            const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
            const bf16x4_t y = __builtin_bit_cast(bf16x4_t, x);
            a[t * 4 + 0] = y[0];
            a[t * 4 + 1] = y[1];
            a[t * 4 + 2] = y[2];
            a[t * 4 + 3] = y[3];
        }
        return a;
    };
    // O^T += V^T P^T for the tile in `stage`: 16 dv blocks x 2 key steps
    constexpr int kPvSteps = kDvBlocks * 2;
    auto pv = [&](int stage, const bf16x8_t (&pf)[2]) __attribute__((always_inline)) {
        const uint8_t* st = smem + stage * kTileBytes;
        bf16x8_t a[kPre];
#pragma unroll
        for (int i = 0; i < kPre; ++i) a[i] = vfrag(st, i);
#pragma unroll
        for (int i = 0; i < kPvSteps; ++i) {
            oacc[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kPre], pf[i & 1], oacc[i >> 1], 0, 0, 0);
            if (i + kPre < kPvSteps) a[i % kPre] = vfrag(st, i + kPre);
        }
    };
    auto tile_max = [&](const f32x16_t& sacc) __attribute__((always_inline)) {
        float mx = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        return xor32_max(mx) * scale_log2;
    };
    // O *= alpha, in place on the accumulators
    auto scale_o = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < kDvBlocks; ++db) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = oacc[db][i];
                agpr_scale(x, alpha);
                oacc[db][i] = x;
            }
        }
    };
    // p = exp2(s - m) as bf16, and the row sum of those bf16 values
    auto exp_part = [&](const f32x16_t& sacc, bf16x8_t (&pf)[2]) __attribute__((always_inline)) {
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

    // ---- pipeline ----
    // Iteration j: wait for tile j (tiles j+1 and j+2 may still be in
    // flight), barrier (retires tile j-1), issue tile j+3 into tile j-1's
    // stage, scores of tile j, the running maximum (O *= 2^(m_old - m_new)
    // if it moved), the softmax of tile j and its PV.
    //
    // The item's keys [kv_lo, kv_hi) are tiles 0 .. n_tiles-1 (kv_lo is a
    // multiple of 32); n_full: tiles every row of the wave sees whole,
    // n_wave: tiles with a key some row of the wave sees
    const int n_tiles = (it.kv_hi - it.kv_lo + kBN - 1) / kBN;
    int nf = wave_lo > it.kv_lo ? (wave_lo - it.kv_lo) / kBN : 0;
    int nw = wave_hi > it.kv_lo ? (wave_hi - it.kv_lo + kBN - 1) / kBN : 0;
    nf = nf < n_tiles ? nf : n_tiles;
    nw = nw < n_tiles ? nw : n_tiles;
    const int n_full = __builtin_amdgcn_readfirstlane(nf);
    const int n_wave = __builtin_amdgcn_readfirstlane(nw);
    // tiles are issued in order; with a paged cache the next tile's table
    // entry is read one issue ahead
    int iss_page = 0;
    if constexpr (kPaged) {
        if (n_tiles > 0) iss_page = page_entry(0);
    }
    auto issue_next = [&](int kt) __attribute__((always_inline)) {
        issue_tile(kt, kt % kStages, iss_page);
        if constexpr (kPaged) {
            if (kt + 1 < n_tiles) iss_page = page_entry(kt + 1);
        }
    };
    auto sync_top = [&](int j) __attribute__((always_inline)) {
        if (j + 2 < n_tiles) wait_vmcnt<2 * kLoadsPerTile>();
        else if (j + 1 < n_tiles) wait_vmcnt<kLoadsPerTile>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (j + 3 < n_tiles) issue_next(j + 3);
    };
    for (int t = 0; t < 3 && t < n_tiles; ++t) issue_next(t);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qf[s] = q_src[2 * s];
    // s_waitcnt vmcnt(0) (expcnt and lgkmcnt fields at their maxima): Q and
    // the first tiles have all landed
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));
    // The empty asm redefines the Q registers after that wait, so the
    // compiler no longer sees loads in flight into them and puts none of its
    // own vmcnt waits in the loop (those would also wait for the ring's
    // tiles in flight, issued as asm it does not count).
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) asm volatile("" : "+v"(qf[s]));

    int j = 0;
    // with_o: O may already hold earlier tiles (false for the first one)
    auto iteration = [&](int jj, auto with_o, auto masked) __attribute__((always_inline)) {
        constexpr bool kO = decltype(with_o)::value;
        sync_top(jj);
        f32x16_t sacc;
        scores(jj, jj % kStages, masked, sacc);
        const float mt = tile_max(sacc);
        // lazy rescale: the maximum moves only when some row's tile maximum
        // exceeds it by more than 2^8 (a wave-uniform decision)
        const bool moved = __any(mt > m_run + kLazyRescale);
        const float m_new = moved ? fmaxf(m_run, mt) : m_run;
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        if constexpr (kO) {
            if (__builtin_expect(moved, 0)) scale_o(alpha);
        }
        bf16x8_t p[2];
        exp_part(sacc, p);
        pv(jj % kStages, p);
    };
    if (n_wave > 0) {
        if (n_full > 0) iteration(0, std::false_type{}, std::false_type{});
        else iteration(0, std::false_type{}, std::true_type{});
        for (j = 1; j < n_full; ++j) iteration(j, std::true_type{}, std::false_type{});
        for (; j < n_wave; ++j) iteration(j, std::true_type{}, std::true_type{});
    }
    // tiles only other waves need: barriers and loads
    for (; j < n_tiles; ++j) sync_top(j);
    wait_vmcnt<0>();

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
    if (wave_rows <= 0) return;
    const float ltot = xor32_sum(l_run);
    // The lane's row and half are recomputed here, by an asm the compiler
    // cannot merge with the one at the top, so no lane-dependent index stays
    // live (or spilled) across the key loop.
    int lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
    const int g_e = lane_e >> 5;
    const int row_e = row_w0 + (lane_e & 31);
    if (row_e >= it.n_rows) return;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.0f;
    const int64_t rho = (int64_t)it.row0 + row_e;
    // a KV split writes its partial state over this item's keys: O (bf16,
    // normalised like a final output) and its LSE (fp32)
    const bool split = it.part >= 0;
    uint16_t* dst = split ? part_o + ((int64_t)it.part * part_rows + rho) * kDv : out + rho * kDv;
#pragma unroll
    for (int db = 0; db < kDvBlocks; ++db) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int dv = db * 32 + grp * 8 + g_e * 4;
            bf16x4_t o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][grp * 4 + e] * inv);
            *reinterpret_cast<bf16x4_t*>(dst + dv) = o4;
        }
    }
    float* lse_dst = split ? part_lse + (int64_t)it.part * part_rows : lse;
    if (g_e == 0 && lse_dst != nullptr)
        lse_dst[rho] = ltot > 0.f ? (m_run + __log2f(ltot)) * kLn2 : -INFINITY;
}

}  // namespace

int prefill_absorbed_block_m() { return kBM; }

hipError_t launch_prefill_absorbed(const LatentItem* items, int64_t n_items, const void* q,
                                   const void* kv, void* out, float* lse, int num_heads,
                                   float sm_scale, hipStream_t stream, const PagedKv* paged,
                                   uint16_t* part_o, float* part_lse, int64_t part_rows) {
    if (n_items <= 0) return hipSuccess;
    if (n_items > 0x7fffffff) return hipErrorInvalidValue;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    const PagedKv pg = paged != nullptr ? *paged : PagedKv{nullptr, 0, 0, 0};
    if (paged != nullptr)
        hipLaunchKernelGGL(prefill_absorbed_kernel<true>, dim3((unsigned)n_items), dim3(kThreads), 0,
                           stream, items, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(kv), static_cast<uint16_t*>(out), lse,
                           num_heads, scale_log2, pg, pg.block_table, part_o, part_lse, part_rows);
    else
        hipLaunchKernelGGL(prefill_absorbed_kernel<false>, dim3((unsigned)n_items), dim3(kThreads), 0,
                           stream, items, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(kv), static_cast<uint16_t*>(out), lse,
                           num_heads, scale_log2, pg, nullptr, part_o, part_lse, part_rows);
    return hipGetLastError();
}

namespace {

// Combine the KV splits of each row (the flash-decoding split of one row's
// keys, merged with the same log-sum-exp weights as merge_state):
//   lse = ln sum_s e^lse_s,  o = sum_s e^(lse_s - lse) o_s;
// splits with lse = -inf carry weight 0; all -inf gives o = 0, lse = -inf.
// One row per wave, 8 dims (16 bytes of each bf16 partial) per lane. The
// wave reads the row's split LSEs in parallel (lane s takes split s) and
// reduces them with cross-lane operations; the weights are then broadcast
// from their lanes, and the partial rows are read a few splits at a time so
// that several loads are in flight.
constexpr int kMergeThreads = 256;
constexpr int kMergeRows = kMergeThreads / 64;
constexpr int kMaxSplits = 64;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

__global__ __launch_bounds__(kMergeThreads) void merge_splits_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse, int splits,
    int64_t rows, uint16_t* __restrict__ out, float* __restrict__ lse) {
    // the row is the same for the whole wave, so a wave returns as a whole
    const int64_t row = (int64_t)blockIdx.x * kMergeRows + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float ls = lane < splits ? part_lse[(int64_t)lane * rows + row] : -INFINITY;
    const float mx = wave_max(ls);
    const float w = (mx == -INFINITY || ls == -INFINITY)
                        ? 0.0f
                        : __builtin_amdgcn_exp2f((ls - mx) * 1.4426950408889634f);
    const float sum = wave_sum(w);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* src = part_o + row * kDv + lane * 8;
    const int64_t split_stride = rows * kDv;
    constexpr int kBatch = 4;
    for (int s0 = 0; s0 < splits; s0 += kBatch) {
        bf16x8_t v[kBatch];
        float ws[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int sk = s0 + k < splits ? s0 + k : splits - 1;
            ws[k] = s0 + k < splits ? __shfl(w, sk) : 0.0f;
            v[k] = ws[k] != 0.0f
                       ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(src + sk * split_stride))
                       : bf16x8_t{};
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += ws[k] * (float)v[k][e];
        }
    }
    const float inv = sum > 0.f ? 1.0f / sum : 0.0f;
    bf16x8_t o8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8_t*>(out + row * kDv + lane * 8) = o8;
    if (lane == 0 && lse != nullptr) lse[row] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
}

}  // namespace

hipError_t launch_merge_splits(const uint16_t* part_o, const float* part_lse, int splits,
                               int64_t rows, void* out, float* lse, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
    const int64_t blocks = (rows + kMergeRows - 1) / kMergeRows;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(merge_splits_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream,
                       part_o, part_lse, splits, rows, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
}

}  // namespace mla
