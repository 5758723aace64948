// Ragged MLA prefill with the KV decompression fused into the attention
// kernel, for gfx950 (CDNA4).
//
// "[DeepseekR1] How ragged prefill manage kv_cache?" (sglang issue 3849)
// asks whether chunked prefill decompresses the 512-dim latent cache (plus
// its 64 RoPE dims) into per-head K/V on every pass. This kernel never
// materialises K/V in HBM: for every 32-key tile it forms
//   K[j, 0:128]   = c_kv[j, :] . W_UK[:, h*128 : h*128+128]
//   K[j, 128:192] = k_rope[j, :]
//   V[j, :]       = c_kv[j, :] . W_UV[:, h*128 : h*128+128]
// in LDS (bf16 MFMA, fp32 accumulation, rounded to bf16 as the separate
// decompression kernel rounds its outputs) and runs the ragged prefill's
// attention on it: S = sm_scale Q K^T over the visible keys (bottom-right
// causal or all), online softmax in fp32, O = P V, natural-log LSE per
// (token, head).
//
// Design (MI355X):
//  * A workgroup serves one head and keeps that head's weights on chip for
//    its whole life: each of its 4 waves (one per SIMD, up to 512 registers)
//    holds the transposed W_UK and W_UV columns of 32 output dims as 64 MFMA
//    operands (256 registers), so W is read from HBM once per workgroup.
//  * Work: the query tiles of 128 rows of all sequences, sorted by the keys
//    they visit, heaviest first; workgroup (head h, part p) takes tiles
//    p, p + P, p + 2P, ... for head h. Workgroups of one part run the same
//    tiles at the same time, and the hardware deals workgroup i to XCD
//    i mod 8, so each XCD's L2 serves one latent stream to all its heads.
//  * Per 32-key tile, the latent rows (32 x 1 KB) and their RoPE dims
//    (32 x 128 B) arrive by global_load_lds_dwordx4 in a 3-stage latent ring
//    and a 4-stage RoPE ring, two tiles ahead. A wave runs 32 k-steps of two
//    MFMAs on one latent fragment read: as the B operand of
//    K^T = W_UK^T c_kv^T and as the A operand of V = c_kv W_UV. In the
//    accumulator layout of v_mfma_f32_32x32x16_bf16 both results, rounded to
//    bf16, already are attention operands: the K^T accumulator holds, per
//    key, the score A operand over a fixed permutation of the wave's 32 NoPE
//    dims (Q is loaded in the same permutation), and the V accumulator holds
//    the PV A operand of the wave's 32 value dims in the key order of the P
//    fragments. LDS only broadcasts them to the other waves: 16-byte writes
//    and reads, rows padded so neither has bank conflicts.
//  * Software pipeline, one barrier per tile: iteration G computes the
//    scores of tile G (K from LDS, its RoPE dims straight from the RoPE
//    ring), its softmax, the decompression of tile G+1 into the other K/V
//    buffer and PV of tile G, then waits for the latent rows of tile G+2,
//    and after the barrier puts tile G+4 in flight. The stream runs on from
//    one query tile into the next; the next tile's Q is loaded during the
//    current tile's last iteration.
//  * The cost of fusion is that every query tile that visits a key tile
//    decompresses it again (64 MFMAs per wave per key tile against the
//    attention's 20).
//  * Online softmax as in the ragged prefill kernel: base 2 with the scale
//    folded into one FMA, lazy rescale (the max is raised only when a tile
//    exceeds it by 2^8), row sum accumulated from the bf16-rounded p.
//  * Keys past a sequence's end load its last row (finite data) and are
//    masked to p = 0; rows with no visible key get O = 0, LSE = -inf.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;                 // query rows per tile
constexpr int kBN = 32;                          // keys per tile
constexpr int kKSteps = kDlat / 16;              // 32 latent k-steps
constexpr int kSSteps = kDqk / 16;               // 12 score k-steps
constexpr int kNopeSteps = kDnope / 16;          // 8 of them over the NoPE dims
constexpr int kCBytes = kBN * kDlat * 2;         // 32 KB of latent rows per tile
constexpr int kRBytes = kBN * kDrope * 2;        // 4 KB of RoPE dims per tile
constexpr int kCStages = 3;
constexpr int kRStages = 4;
constexpr int kKRow = kDnope * 2 + 16;           // K buffer row: 128 dims + pad (272 B)
constexpr int kVRow = kBN * 2 + 16;              // V^T buffer row: 32 keys + pad (80 B)
constexpr int kKBuf = kBN * kKRow;               // 8.5 KB
constexpr int kVBuf = kDvo * kVRow;              // 10 KB
constexpr int kROff = kCStages * kCBytes;
constexpr int kKOff = kROff + kRStages * kRBytes;
constexpr int kVOff = kKOff + 2 * kKBuf;
constexpr int kLds = kVOff + 2 * kVBuf;          // 149 KB
constexpr int kCLoads = kCBytes / 1024 / kWaves; // 8 latent rows per wave per tile
constexpr int kLoadsPerTile = kCLoads + 1;       // + 1 KB of RoPE dims
constexpr int kWRowB = kDnope * 2;               // 256 B: one latent row of a head's W slice
constexpr int kWRound = 128;                     // latent rows per W load round
constexpr int kPrefetch = 4;                     // latent fragments read ahead
constexpr float kLazyRescale = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;
// s_waitcnt immediate that waits for vmcnt = 0 only (gfx9 encoding)
constexpr int kVmcnt0 = (0x7 << 4) | (0xf << 8);
static_assert(2 * kWRound * kWRowB <= kROff, "a W round fits in the latent ring");
static_assert(kLds <= 160 * 1024, "LDS budget of one CU");

// 16-byte chunk slots: latent rows (64 chunks, XOR by row), RoPE rows (8
// chunks, XOR by row / 2), W rows (16 chunks, XOR by row % 4 in groups of 4)
__device__ __forceinline__ int cslot(int t, int c) { return c ^ (t & 15); }
__device__ __forceinline__ int rslot(int t, int c) { return c ^ ((t >> 1) & 7); }
__device__ __forceinline__ int wslot(int r, int c) { return c ^ ((r & 3) << 2); }

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

// One 16-byte-per-lane global -> LDS load (lane l's 16 bytes land at
// lds_dst + 16 l; the global address is the wave-uniform sbase plus the
// lane's voff), issued as inline asm so the compiler does not wait for it
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

__device__ __forceinline__ bf16x8_t to_bf16x8(const f32x16_t& a, int half) {
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)a[8 * half + e];
    return r;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decompress_prefill_kernel(const WorkItem* __restrict__ tiles, int n_tiles, int n_busy,
                               int parts, const uint16_t* __restrict__ q,
                               const uint16_t* __restrict__ c_kv,
                               const uint16_t* __restrict__ k_rope,
                               const uint16_t* __restrict__ w_uk,
                               const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
                               float* __restrict__ lse, int num_heads, float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int H = num_heads;
    const int head = blockIdx.x / parts;
    const int part = blockIdx.x - head * parts;
    const int my_row = wave * 32 + l32;              // this lane's row in a query tile

    // Tiles below n_busy see keys; this workgroup's are part + j * parts.
    const int n_mine = n_busy > part ? (n_busy - part + parts - 1) / parts : 0;

    // Tiles without a visible key (sorted last): O = 0, LSE = -inf.
    for (int k = part + n_mine * parts; k < n_tiles; k += parts) {
        if (my_row < tiles[k].n_rows) {
            const int64_t orow = (int64_t)(tiles[k].q_row0 + my_row) * H + head;
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + orow * kDvo + 64 * g);
#pragma unroll
            for (int c = 0; c < 8; ++c) dst[c] = u32x4_t{0u, 0u, 0u, 0u};
            if (g == 0 && lse != nullptr) lse[orow] = -INFINITY;
        }
    }
    if (n_mine == 0) return;

    // ---- this wave's transposed W_UK / W_UV columns into registers ----
    // Round rnd stages latent rows 128 rnd .. +128 of both slices in LDS:
    // matrix m at m * 32 KB, row r at r * 256 B, 16-byte chunk c at slot
    // wslot(r, c). Waves 0-1 load W_UK, waves 2-3 W_UV (16 blocks of 4 rows
    // each). A fragment of k-step ks: lane (g, h = bit 4, r = bits 2-3,
    // q = bits 0-1) supplies latent row 16 ks + 8 g + 4 t + r, dims
    // 32 wave + 16 h + 4 q .. +4 (two transposing reads, t = 0, 1), and lane
    // 16 h + j of each half receives dim 32 wave + 16 h + j with its 8
    // k-slots in natural latent order: the A operand of W^T and, as the same
    // registers, the B operand of W.
    bf16x8_t wk[kKSteps], wv[kKSteps];
    {
        const int mat = wave >> 1;
        const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(mat == 0 ? w_uk : w_uv) +
                              (int64_t)head * kWRowB;
        const uint32_t wstride = (uint32_t)H * kWRowB;
        uint32_t off[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int row = 4 * (16 * (wave & 1) + j) + (lane >> 4);
            off[j] = (uint32_t)row * wstride + (uint32_t)wslot(row, lane & 15) * 16;
        }
        int a_off;
        {
            const int tr_h = (lane >> 4) & 1;
            const int tr_r = (lane & 15) >> 2;
            const int tr_q = lane & 3;
            const int row = 8 * g + tr_r;
            const int chunk = 4 * wave + 2 * tr_h + (tr_q >> 1);
            a_off = row * kWRowB + wslot(row, chunk) * 16 + (tr_q & 1) * 8;
        }
#pragma unroll
        for (int rnd = 0; rnd < kDlat / kWRound; ++rnd) {
            const uint8_t* rb = wsrc + (int64_t)rnd * kWRound * wstride;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                dma16(rb, off[j], smem + mat * (kWRound * kWRowB) + (16 * (wave & 1) + j) * 1024);
            wait_vmcnt<0>();
            __syncthreads();
#pragma unroll
            for (int ksl = 0; ksl < kWRound / 16; ++ksl) {
                const int ks = rnd * (kWRound / 16) + ksl;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const uint8_t* p = smem + m * (kWRound * kWRowB) + a_off + (16 * ksl + 4 * t) * kWRowB;
                        const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
                        const bf16x4_t y = __builtin_bit_cast(bf16x4_t, x);
                        bf16x8_t& dst = m == 0 ? wk[ks] : wv[ks];
                        dst[4 * t + 0] = y[0];
                        dst[4 * t + 1] = y[1];
                        dst[4 * t + 2] = y[2];
                        dst[4 * t + 3] = y[3];
                    }
                }
            }
            __syncthreads();
        }
    }

    // ---- latent stream: issue cursor ----
    // Global tile G of this workgroup = key tile kt of its j-th query tile;
    // its latent rows go to latent stage G % 3, its RoPE dims to RoPE stage
    // G % 4. Wave w loads latent rows 8 w .. 8 w + 7 (1 KB each, chunk c at
    // slot cslot) and RoPE rows 8 w .. 8 w + 7 (128 B each, chunk c at slot
    // rslot). Keys at or past kv_len load the last key's row; the DMA base
    // stays wave-uniform and the RoPE row clamp goes into the lane offset.
    int iss_g = 0, iss_j = 0, iss_kt = 0;
    int iss_nk = 0, iss_kvstart = 0, iss_kvlen = 0;
    auto iss_load = [&]() {
        const int k = part + iss_j * parts;
        iss_nk = (tiles[k].kv_hi + kBN - 1) / kBN;
        iss_kvstart = tiles[k].kv_start;
        iss_kvlen = tiles[k].kv_len;
    };
    iss_load();
    auto issue_next = [&]() {
        uint8_t* cs = smem + (iss_g % kCStages) * kCBytes;
        uint8_t* rs = smem + kROff + (iss_g % kRStages) * kRBytes;
        const int key0 = iss_kt * kBN;
        const int last = iss_kvlen - 1;
        const bool full = key0 + kBN - 1 <= last;
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) {
            const int rr = kCLoads * wave + j;
            const int key = full || key0 + rr <= last ? key0 + rr : last;
            dma16(c_kv + (int64_t)(iss_kvstart + key) * kDlat, (uint32_t)cslot(rr, lane) * 16,
                  cs + rr * 1024);
        }
        {
            const int t = 8 * wave + (lane >> 3);
            const int key = full || key0 + t <= last ? key0 + t : last;
            dma16(k_rope + (int64_t)(iss_kvstart + key0) * kDrope,
                  (uint32_t)(key - key0) * (kDrope * 2) + (uint32_t)rslot(t, lane & 7) * 16,
                  rs + wave * 1024);
        }
        ++iss_g;
        if (++iss_kt == iss_nk) {
            iss_kt = 0;
            if (++iss_j < n_mine) iss_load();
        }
    };

    // ---- decompression of one latent stage into one K / V^T buffer ----
    // K buffer: row = key (272 B); the K^T accumulator's registers 8 u .. 8 u
    // + 7 (u = 0, 1) of lane (key, g) go to bytes 32 (2 wave + u) + 16 g.
    // V^T buffer: row = value dim (80 B); the V accumulator's registers
    // 8 u .. 8 u + 7 of lane (dim 32 wave + l32, g) go to bytes 16 (2 u + g).
    const int c_rd = l32 * 1024;
    auto decompress = [&](int stage, int buf) {
        const uint8_t* cs = smem + stage * kCBytes;
        bf16x8_t cf[kPrefetch];
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u)
            cf[u] = *reinterpret_cast<const bf16x8_t*>(cs + c_rd + cslot(l32, 2 * u + g) * 16);
        f32x16_t acc_k = f32x16_t{}, acc_v = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8_t b = cf[ks % kPrefetch];
            if (ks + kPrefetch < kKSteps)
                cf[ks % kPrefetch] = *reinterpret_cast<const bf16x8_t*>(
                    cs + c_rd + cslot(l32, 2 * (ks + kPrefetch) + g) * 16);
            acc_k = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wk[ks], b, acc_k, 0, 0, 0);
            acc_v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, wv[ks], acc_v, 0, 0, 0);
        }
        uint8_t* kb = smem + kKOff + buf * kKBuf + l32 * kKRow + 64 * wave + 16 * g;
        uint8_t* vb = smem + kVOff + buf * kVBuf + (32 * wave + l32) * kVRow + 16 * g;
        *reinterpret_cast<bf16x8_t*>(kb) = to_bf16x8(acc_k, 0);
        *reinterpret_cast<bf16x8_t*>(kb + 32) = to_bf16x8(acc_k, 1);
        *reinterpret_cast<bf16x8_t*>(vb) = to_bf16x8(acc_v, 0);
        *reinterpret_cast<bf16x8_t*>(vb + 32) = to_bf16x8(acc_v, 1);
    };

    // ---- current query tile ----
    // Q fragments (B operand): NoPE step s holds, in k-slots 8 g + 4 u + e,
    // dim 32 (s / 2) + 16 (s % 2) + 8 u + 4 g + e (the K buffer's order);
    // RoPE step 8 + r holds dims 128 + 16 r + 8 g .. +8.
    bf16x8_t qf[kSSteps];
    auto load_q = [&](int q_row0, int n_rows) {
        const int r = my_row < n_rows ? my_row : n_rows - 1;
        const uint16_t* src = q + ((int64_t)(q_row0 + r) * H + head) * kDqk;
#pragma unroll
        for (int s = 0; s < kNopeSteps; ++s) {
            const int d0 = 32 * (s >> 1) + 16 * (s & 1) + 4 * g;
            const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(src + d0);
            const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(src + d0 + 8);
            qf[s] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int s = kNopeSteps; s < kSSteps; ++s)
            qf[s] = *reinterpret_cast<const bf16x8_t*>(src + kDnope + 16 * (s - kNopeSteps) + 8 * g);
    };

    // fields of the current query tile (wave-uniform)
    int cur_j = 0;
    int cur_q_row0 = tiles[part].q_row0;
    int cur_n_rows = tiles[part].n_rows;
    int cur_nk = (tiles[part].kv_hi + kBN - 1) / kBN;
    int my_lim = lim_of(my_row, tiles[part].diag0, tiles[part].kv_len);

    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

    const int k_rd = l32 * kKRow + 16 * g;
    const int r_rd = l32 * (kDrope * 2);
    auto scores = [&](int kt, int buf, int rstage, f32x16_t& sacc) {
        const uint8_t* kb = smem + kKOff + buf * kKBuf + k_rd;
        const uint8_t* rs = smem + kROff + rstage * kRBytes + r_rd;
        sacc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kNopeSteps; ++s) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kb + 32 * s);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
        }
#pragma unroll
        for (int s = kNopeSteps; s < kSSteps; ++s) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                rs + rslot(l32, 2 * (s - kNopeSteps) + g) * 16);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
        }
        const int key0 = kt * kBN;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = key0 + (i >> 2) * 8 + g * 4 + (i & 3);
            sacc[i] = key < my_lim ? sacc[i] : -INFINITY;
        }
    };
    auto pv = [&](int buf, const bf16x8_t (&pf)[2]) {
        const uint8_t* vb = smem + kVOff + buf * kVBuf + l32 * kVRow + 16 * g;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vb + 32 * db * kVRow + 32 * mm);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[mm], oacc[db], 0, 0, 0);
            }
        }
    };
    auto store_out = [&]() {
        const float ltot = xor32_sum(l_run);
        if (my_row >= cur_n_rows) return;
        const float inv = ltot > 0.f ? 1.0f / ltot : 0.0f;
        const int64_t orow = (int64_t)(cur_q_row0 + my_row) * H + head;
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

    // ---- prologue: tiles 0..2 in flight, Q, decompression of tile 0 ----
    for (int t = 0; t < 3 && iss_j < n_mine; ++t) issue_next();
    load_q(cur_q_row0, cur_n_rows);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    decompress(0, 0);
    __syncthreads();
    if (iss_j < n_mine) issue_next();

    int kt = 0;
    for (int G = 0;; ++G) {
        const bool last_kt = kt + 1 == cur_nk;
        const bool more_q = cur_j + 1 < n_mine;
        f32x16_t sacc;
        scores(kt, G & 1, G % kRStages, sacc);
        const int nxt = part + (cur_j + 1) * parts;    // next query tile (if more_q)
        if (last_kt && more_q) load_q(tiles[nxt].q_row0, tiles[nxt].n_rows);   // after this tile's scores
        float mt = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sacc[i]);
        mt = xor32_max(mt) * scale_log2;
        if (__builtin_expect(__any(mt > m_run + kLazyRescale), 0)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
        }
        bf16x8_t pf[2];
        {
            const float msub = m_run == -INFINITY ? 0.0f : m_run;
            float lsum = l_run;
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mm * 8 + e], scale_log2, -msub));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mm * 8 + e + 1], scale_log2, -msub));
                    const bf16x2_t pk = {(__bf16)p0, (__bf16)p1};
                    pf[mm][e] = pk[0];
                    pf[mm][e + 1] = pk[1];
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes, lsum, false);
                }
            }
            l_run = lsum;
        }
        if (!last_kt || more_q) decompress((G + 1) % kCStages, (G + 1) & 1);
        pv(G & 1, pf);
        if (last_kt) {
            store_out();
            // stores and the next Q loads are younger than the latent rows
            // of tile G+2: drain everything
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
        } else if (iss_g >= G + 4) {
            wait_vmcnt<kLoadsPerTile>();    // tile G+3 may stay in flight
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        if (iss_j < n_mine) issue_next();
        if (last_kt) {
            if (!more_q) break;
            ++cur_j;
            cur_q_row0 = tiles[nxt].q_row0;
            cur_n_rows = tiles[nxt].n_rows;
            cur_nk = (tiles[nxt].kv_hi + kBN - 1) / kBN;
            my_lim = lim_of(my_row, tiles[nxt].diag0, tiles[nxt].kv_len);
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
            m_run = -INFINITY;
            l_run = 0.f;
            kt = 0;
        } else {
            ++kt;
        }
    }
    wait_vmcnt<0>();
}

}  // namespace

int decompress_prefill_block_m() { return kBM; }

hipError_t launch_decompress_prefill(const WorkItem* tiles, int64_t n_tiles, int64_t n_busy,
                                     const void* q, const void* c_kv, const void* k_rope,
                                     const void* w_uk, const void* w_uv, void* out, float* lse,
                                     int num_heads, float sm_scale, hipStream_t stream) {
    if (n_tiles <= 0) return hipSuccess;
    if (n_tiles > 0x7fffffff || n_busy < 0 || n_busy > n_tiles || num_heads < 1 ||
        num_heads > 65535)
        return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus <= 0) cus = 256;
    // one workgroup per CU (its LDS allows no more): enough parts per head
    // to fill the chip, at most one per busy tile
    int64_t parts = cus / num_heads;
    if (parts > n_busy) parts = n_busy;
    if (parts < 1) parts = 1;
    const int64_t blocks = parts * num_heads;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(decompress_prefill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       tiles, (int)n_tiles, (int)n_busy, (int)parts,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c_kv),
                       static_cast<const uint16_t*>(k_rope), static_cast<const uint16_t*>(w_uk),
                       static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out), lse,
                       num_heads, scale_log2);
    return hipGetLastError();
}

}  // namespace mla
