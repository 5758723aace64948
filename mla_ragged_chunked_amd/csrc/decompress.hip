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
// Design (MI355X): weight-stationary.
//  * A workgroup owns one block of 2 heads (256 output dims) of W_UK or W_UV
//    and a contiguous range of tokens. Its 8 waves (two per SIMD) each keep
//    the transposed weights of 32 output dims for all 512 latent dims in
//    registers for the whole kernel (32 MFMA A operands, 128 VGPRs), loaded
//    once through LDS with transposing reads.
//  * The latent cache streams through a 4-stage LDS ring in tiles of 32
//    tokens (32 KB of c_kv + 4 KB of k_rope per tile) loaded straight from
//    HBM with global_load_lds_dwordx4; every wave reads the whole tile as
//    the B operand (c_kv rows XOR-swizzled by token: conflict-free 16-byte
//    reads) and runs 32 MFMAs (v_mfma_f32_32x32x16_bf16, C^T[n][t]).
//  * The grid is one round: 2 x ceil(H/2) head blocks x (CUs / head blocks)
//    token ranges, so every weight is read from HBM once per token range
//    and the operand traffic is ~4.4 GB at the DeepSeek shape (a 256 x 256
//    output-tile GEMM reads ~8.6 GB).
//  * Outputs leave straight from the accumulator: in a 32x32 block lane
//    (token, half g) holds dims 8q + 4g + e; one v_permlane32_swap per
//    register pair gives each lane 8 consecutive dims, so every store is
//    16 bytes per lane and 32 contiguous bytes per token. The head's four
//    waves also copy the tile's k_rope into dims 128..191 (8 tokens x 128 B
//    per store).
//  * Two waves per SIMD let one wave's stores overlap the other's MFMAs.
//    Measured on MI355X, MFMA work and a heavy HBM write stream do not
//    overlap chip-wide (MFMA-only and store-only workgroups sharing a grid
//    take nearly the sum of their separate times), which sets the floor of
//    this kernel near the sum of its MFMA time and its 2.7 GB of writes.
//  * Rows past the last token load the last token (finite) and are not
//    stored; an odd head count leaves the second head's waves of the last
//    block idle.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kNW = 32;                         // output dims per wave (one 32-dim block)
constexpr int kNB = kWaves * kNW;               // 256 output dims per workgroup = 2 heads
constexpr int kKSteps = kDlat / 16;             // 32
constexpr int kTT = 32;                         // tokens per c_kv tile
constexpr int kCRowB = kDlat * 2;               // 1 KB: one token's latent
constexpr int kCBytes = kTT * kCRowB;           // 32 KB
constexpr int kRBytes = kTT * kDrope * 2;       // 4 KB of k_rope per tile
constexpr int kStage = kCBytes + kRBytes;       // 36 KB
constexpr int kStages = 4;                      // 144 KB ring
constexpr int kLds = kStages * kStage;
constexpr int kWRowB = kNB * 2;                 // 512 B: one latent row of the W block
constexpr int kWRound = 128;                    // latent rows of W per load round (64 KB)
static_assert(kWRound * kWRowB <= kLds, "a W round fits in the ring");
constexpr int kCLoads = kCBytes / 1024 / kWaves;    // 4 c_kv rows per wave per tile
constexpr int kRopeWaves = kRBytes / 1024;          // waves 0..3 also load 1 KB of k_rope
constexpr int kPrefetch = 4;                        // B fragments read ahead of their MFMA

// 16-byte chunk slot of chunk c in c_kv row t (64 chunks per 1 KB row)
__device__ __forceinline__ int cslot(int t, int c) { return c ^ (t & 15); }
// 16-byte chunk slot of chunk c in W block row r (32 chunks per 512 B row)
__device__ __forceinline__ int wslot(int r, int c) { return c ^ ((r & 3) << 2); }

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

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decompress_kernel(const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_rope,
                       const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                       int num_tokens, int num_heads, int splits, int tiles_per,
                       uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int H = num_heads;
    const int blocks_per_mat = (H + 1) >> 1;          // 2-head blocks of K (and of V)
    const int nblk = blockIdx.x / splits;
    const int split = blockIdx.x - nblk * splits;
    const bool is_v = nblk >= blocks_per_mat;
    const int head0 = 2 * (is_v ? nblk - blocks_per_mat : nblk);
    const int n_heads = H - head0 < 2 ? H - head0 : 2;
    const int my_head = head0 + (wave >> 2);          // waves 0-3: first head, 4-7: second
    const int nsub = (wave & 3) * kNW;                // this wave's first dim in its head
    const bool wave_active = (wave >> 2) < n_heads;
    const uint16_t* w = is_v ? w_uv : w_uk;
    const int n_tiles_all = (num_tokens + kTT - 1) / kTT;
    const int tile0 = split * tiles_per;
    int n_tiles = n_tiles_all - tile0;
    n_tiles = n_tiles < 0 ? 0 : (n_tiles > tiles_per ? tiles_per : n_tiles);

    // ---- this wave's W^T fragments into registers, in 4 rounds of 128 latent rows ----
    // W block row c = W[c][head0*128 .. head0*128 + 256) (512 B; a missing
    // second head reads the first head's columns instead). A fragment of
    // k-step ks: lane (g, h = bit 4, r = bits 2-3, q = bits 0-1) supplies
    // latent row 16 ks + 8 g + 4 t + r, dims 32 wave + 16 h + 4 q .. +4 (two
    // transposing reads, t = 0, 1), and lane 16 h + j of each half receives
    // dim 32 wave + 16 h + j with its 8 k-slots in natural latent order.
    bf16x8_t wa[kKSteps];
    {
        const int head_b = n_heads > 1 ? head0 + 1 : head0;
        uint32_t off[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // DMA block b = 8 wave + j (1 KB = 2 rows of 512 B): row 2 b + lane/32
            const int row = 2 * (8 * wave + j) + (lane >> 5);
            const int c = wslot(row, lane & 31);
            const int hsel = c >= 16 ? head_b : head0;
            off[j] = (uint32_t)row * (uint32_t)(H * kDnope * 2) + (uint32_t)(hsel * kDnope * 2) + (c & 15) * 16;
        }
        int a_off;
        {
            const int tr_h = (lane >> 4) & 1;
            const int tr_r = (lane & 15) >> 2;
            const int tr_q = lane & 3;
            const int row = 8 * g + tr_r;
            const int chunk = (kNW * wave + 16 * tr_h + 4 * tr_q) / 8;
            a_off = row * kWRowB + wslot(row, chunk) * 16 + (tr_q & 1) * 8;
        }
        const uint8_t* wbase = reinterpret_cast<const uint8_t*>(w);
#pragma unroll
        for (int rnd = 0; rnd < kDlat / kWRound; ++rnd) {
            const uint8_t* rb = wbase + (int64_t)rnd * kWRound * H * kDnope * 2;
#pragma unroll
            for (int j = 0; j < 8; ++j) dma16(rb, off[j], smem + (8 * wave + j) * 1024);
            wait_vmcnt<0>();
            __syncthreads();
#pragma unroll
            for (int ksl = 0; ksl < kWRound / 16; ++ksl) {
                const int ks = rnd * (kWRound / 16) + ksl;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint8_t* p = smem + a_off + (16 * ksl + 4 * t) * kWRowB;
                    const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
                    const bf16x4_t y = __builtin_bit_cast(bf16x4_t, x);
                    wa[ks][4 * t + 0] = y[0];
                    wa[ks][4 * t + 1] = y[1];
                    wa[ks][4 * t + 2] = y[2];
                    wa[ks][4 * t + 3] = y[3];
                }
            }
            __syncthreads();
        }
    }

    // ---- stream 32-token tiles of c_kv (and k_rope) through the ring ----
    const int last_tok = num_tokens - 1;
    const bool rope_loader = wave < kRopeWaves;
    // DMA of tile i: this wave's 4 c_kv rows (rows 4 wave .. +3, 1 KB each;
    // slot l holds chunk cslot(row, l)); waves 0-3 also 1 KB of k_rope
    // (tokens 8 wave .. +7, 128 B each). Rows past the last token load the
    // last token; the base stays wave-uniform and the clamped per-lane token
    // goes into the lane offset.
    auto issue = [&](int i) {
        uint8_t* cs = smem + (i % kStages) * kStage;
        const int tok0 = (tile0 + i) * kTT;
        const bool full = tok0 + kTT - 1 <= last_tok;
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) {
            const int row = kCLoads * wave + j;
            const int t = full || tok0 + row <= last_tok ? tok0 + row : last_tok;
            dma16(c_kv + (int64_t)t * kDlat, cslot(row, lane) * 16, cs + row * 1024);
        }
        if (rope_loader) {
            const int rt = tok0 + 8 * wave + (lane >> 3);
            const int t = full || rt <= last_tok ? rt : last_tok;
            dma16(k_rope + (int64_t)tok0 * kDrope, (uint32_t)(t - tok0) * (kDrope * 2) + (lane & 7) * 16,
                  cs + kCBytes + wave * 1024);
        }
    };

    const int b_base = l32 * kCRowB;                  // B fragment: token row l32, chunk 2 ks + g
    const int out_dim = is_v ? kDvo : kDqk;
    uint16_t* dst_base = is_v ? v_out : k_out;

    // Vector-memory ops of a wave, in issue order: the DMA of tiles 0, 1 and
    // 2, then per iteration i the DMA of tile i+3 (D = 4 ops, 5 for waves
    // 0-3) at its top and the stores S(i) of tile i at its end (2 output
    // stores; K blocks 1 more of k_rope). Every op but the last tile's has an
    // active lane, so the counts are exact: after tile i's DMA come DMA(1),
    // DMA(2) (i = 0); DMA(2), DMA(3), S(0) (i = 1); DMA(3), S(0), DMA(4),
    // S(1) (i = 2); S(i-3), DMA(i+1), S(i-2), DMA(i+2), S(i-1) (i >= 3). The
    // wait for tile i leaves those in flight; near the end (i + 2 >= tiles)
    // it waits for everything.
    auto wait_tile = [&](int i) {
        if (i + 2 >= n_tiles) { wait_vmcnt<0>(); return; }
        const int st_ = !wave_active ? 0 : (is_v ? 2 : 3);
        const int d_ = rope_loader ? kCLoads + 1 : kCLoads;
        const int after = 2 * d_ + (i < 3 ? i : 3) * st_;
        switch (after) {
            case 8: wait_vmcnt<8>(); break;
            case 10: wait_vmcnt<10>(); break;
            case 11: wait_vmcnt<11>(); break;
            case 12: wait_vmcnt<12>(); break;
            case 13: wait_vmcnt<13>(); break;
            case 14: wait_vmcnt<14>(); break;
            case 15: wait_vmcnt<15>(); break;
            case 16: wait_vmcnt<16>(); break;
            case 17: wait_vmcnt<17>(); break;
            case 18: wait_vmcnt<18>(); break;
            case 19: wait_vmcnt<19>(); break;
            default: wait_vmcnt<0>(); break;
        }
    };
    auto pack4 = [&](const f32x16_t& a, int q) {
        const bf16x4_t o = {(__bf16)a[4 * q], (__bf16)a[4 * q + 1], (__bf16)a[4 * q + 2], (__bf16)a[4 * q + 3]};
        return __builtin_bit_cast(u32x2_t, o);
    };

    if (n_tiles > 0) issue(0);
    if (n_tiles > 1) issue(1);
    if (n_tiles > 2) issue(2);
    for (int i = 0; i < n_tiles; ++i) {
        wait_tile(i);
        __syncthreads();
        if (i + 3 < n_tiles) issue(i + 3);   // into tile i-1's stage, retired by the barrier
        if (!wave_active) continue;
        const uint8_t* st = smem + (i % kStages) * kStage;
        bf16x8_t bq[kPrefetch];
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u)
            bq[u] = *reinterpret_cast<const bf16x8_t*>(st + b_base + cslot(l32, 2 * u + g) * 16);
        f32x16_t acc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8_t b = bq[ks % kPrefetch];
            if (ks + kPrefetch < kKSteps)
                bq[ks % kPrefetch] =
                    *reinterpret_cast<const bf16x8_t*>(st + b_base + cslot(l32, 2 * (ks + kPrefetch) + g) * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[ks], b, acc, 0, 0, 0);
        }
        // v_permlane32_swap exchanges the upper 32 lanes of its first operand
        // with the lower 32 lanes of its second: lane g = 0 ends with dims
        // 16 pr + 0..7, lane g = 1 with 16 pr + 8..15
        const int tok0 = (tile0 + i) * kTT;
        const int t = tok0 + l32;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            u32x2_t y = pack4(acc, 2 * pr);       // dims 16 pr + 4 g .. +4
            u32x2_t x = pack4(acc, 2 * pr + 1);   // dims 16 pr + 8 + 4 g .. +4
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const auto sw = __builtin_amdgcn_permlane32_swap(y[r], x[r], false, false);
                y[r] = sw[0];
                x[r] = sw[1];
            }
            if (t <= last_tok)
                *reinterpret_cast<u32x4_t*>(dst_base + ((int64_t)t * H + my_head) * out_dim + nsub +
                                            16 * pr + 8 * g) = u32x4_t{y[0], y[1], x[0], x[1]};
        }
        if (!is_v) {
            // k_rope into dims 128..191 of this wave's head: the head's 4 waves
            // take 8 tokens each
            const int tl = 8 * (wave & 3) + (lane >> 3);
            const int c = lane & 7;
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(st + kCBytes + tl * (kDrope * 2) + c * 16);
            if (tok0 + tl <= last_tok)
                *reinterpret_cast<u32x4_t*>(k_out + ((int64_t)(tok0 + tl) * H + my_head) * kDqk + kDnope + 8 * c) = x;
        }
    }
    wait_vmcnt<0>();
}

}  // namespace

hipError_t launch_decompress(const void* c_kv, const void* k_rope, const void* w_uk,
                             const void* w_uv, int64_t num_tokens, int num_heads, void* k_out,
                             void* v_out, hipStream_t stream) {
    if (num_tokens <= 0) return hipSuccess;
    if (num_tokens > 0x7fffffff || num_heads > 65535) return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus <= 0) cus = 256;
    // one round: every workgroup keeps its weights for its whole token range
    const int64_t nblk = 2 * (int64_t)((num_heads + 1) / 2);
    const int64_t n_tiles = (num_tokens + kTT - 1) / kTT;
    int64_t splits = cus / nblk;
    if (splits < 1) splits = 1;
    if (splits > n_tiles) splits = n_tiles;
    const int64_t tiles_per = (n_tiles + splits - 1) / splits;
    const int64_t blocks = nblk * splits;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decompress_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(k_rope),
                       static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
                       (int)num_tokens, num_heads, (int)splits, (int)tiles_per,
                       static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
    return hipGetLastError();
}

}  // namespace mla
