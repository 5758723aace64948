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
// Design (MI355X):
//  * One workgroup = 256 tokens x 2 heads (256 output dims) of either K or V
//    (grid.z), 4 waves of 128 dims x 128 tokens, one wave per SIMD with its
//    256 fp32 accumulators in AGPRs. Per MFMA a wave reads 512 B of LDS.
//  * The product is computed transposed, C^T[n][t] = sum_c W[c][n] c_kv[t][c]
//    with v_mfma_f32_32x32x16_bf16 (A = W^T, B = c_kv^T), so each accumulator
//    lane owns one token and runs of four consecutive output dims, written
//    as 8-byte stores (L2 merges them into whole lines).
//  * Operands stream through a 4-stage LDS ring of 32-latent slices, loaded
//    straight from HBM with global_load_lds_dwordx4 (no VGPR staging), one
//    barrier per slice, three slices in flight. W keeps its natural layout
//    (latent rows of 512 B with an XOR swizzle of the 16-byte chunks) and
//    its A fragments are read with ds_read_b64_tr_b16; c_kv rows (64 B per
//    slice) are swizzled so the B fragment reads are conflict free.
//  * Measured on MI355X the kernel is bound by streaming the operands into
//    LDS and by the output stores, not by the MFMAs (removing the MFMAs
//    leaves the time unchanged); the output is 2.7 GB at the DeepSeek shape.
//  * K workgroups also copy k_rope into dims 128..191 of both heads.
//  * Tokens past the end load the last valid row and are not stored; an odd
//    head count leaves the second half of the last pair idle.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTT = 256;                    // tokens per tile
constexpr int kHeads = 2;                   // heads per tile
constexpr int kNT = kHeads * kDnope;        // 256 output dims per tile
constexpr int kKC = 32;                     // latent dims per slice
constexpr int kCBytes = kTT * kKC * 2;      // 16 KB: c_kv rows of 64 B
constexpr int kWBytes = kKC * kNT * 2;      // 16 KB: W rows of 512 B
constexpr int kStage = kCBytes + kWBytes;   // 32 KB
constexpr int kStages = 4;
constexpr int kSlices = kDlat / kKC;        // 16
constexpr int kCLoads = kCBytes / 1024 / kWaves;   // 4 DMA blocks per wave
constexpr int kWLoads = kWBytes / 1024 / kWaves;   // 4
constexpr int kLoadsPerSlice = kCLoads + kWLoads;
static_assert(kCLoads * kWaves * 1024 == kCBytes && kWLoads * kWaves * 1024 == kWBytes, "DMA split");

// 16-byte chunk slot of c_kv chunk c (0..3) in token row t
__device__ __forceinline__ int cslot(int t, int c) { return c ^ ((t >> 2) & 3); }
// 16-byte chunk slot of W chunk c (0..31) in latent row r
__device__ __forceinline__ int wslot(int r, int c) { return c ^ ((r & 3) << 2); }

// One 16-byte-per-lane global -> LDS load (lane l's 16 bytes land at
// lds_dst + 16 l), issued as inline asm so the compiler does not wait for
// it before LDS reads; completion is awaited with wait_vmcnt before the
// barrier that publishes a slice. Nothing else in this kernel uses M0.
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

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decompress_kernel(const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_rope,
                       const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                       int num_tokens, int num_heads, uint16_t* __restrict__ k_out,
                       uint16_t* __restrict__ v_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int t0 = blockIdx.x * kTT;
    const int head0 = blockIdx.y * kHeads;
    const bool is_v = blockIdx.z == 1;
    const uint16_t* w = is_v ? w_uv : w_uk;
    const int H = num_heads;
    // heads of this tile that exist (the second may not, for odd H)
    const int n_heads = H - head0 < kHeads ? H - head0 : kHeads;
    const int wn = wave & 1;     // head head0 + wn: dims [128 wn, +128) of the tile
    const int wt = wave >> 1;    // tokens [128 wt, +128)
    const bool wave_active = wn < n_heads;

    // ---- DMA addressing (per lane, per slice: base + 16-byte chunk) ----
    // c_kv block j of this wave: tile rows 16 (4 wave + j) + lane/4, LDS slot
    // lane%4 holds global chunk cslot(row, lane%4) of the slice.
    uint32_t c_off[kCLoads];
#pragma unroll
    for (int j = 0; j < kCLoads; ++j) {
        const int row = 16 * (kCLoads * wave + j) + (lane >> 2);
        int t = t0 + row;
        t = t < num_tokens ? t : num_tokens - 1;
        c_off[j] = (uint32_t)(t - t0) * (kDlat * 2) + cslot(row, lane & 3) * 16;
    }
    // W block j of this wave: latent rows 2 (4 wave + j) + lane/32 of the
    // slice, LDS slot lane%32 holds global chunk wslot(row, lane%32).
    const int head_w1 = n_heads > 1 ? head0 + 1 : head0;   // clamp a missing head
    uint32_t w_off[kWLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
        const int row = 2 * (kWLoads * wave + j) + (lane >> 5);
        const int c = wslot(row, lane & 31);                    // 0..31 over the 2 heads
        const int hsel = c >= 16 ? head_w1 : head0;
        w_off[j] = (uint32_t)row * (uint32_t)(H * kDnope * 2) + (uint32_t)(hsel * kDnope * 2) + (c & 15) * 16;
    }
    const uint8_t* cbase = reinterpret_cast<const uint8_t*>(c_kv + (int64_t)t0 * kDlat);
    const uint8_t* wbase = reinterpret_cast<const uint8_t*>(w);
    auto issue = [&](int slice) {
        uint8_t* cs = smem + (slice % kStages) * kStage;
        uint8_t* ws = cs + kCBytes;
        const uint8_t* cb = cbase + slice * kKC * 2;
        const uint8_t* wb = wbase + (int64_t)slice * kKC * H * kDnope * 2;
#pragma unroll
        for (int j = 0; j < kCLoads; ++j) dma16(cb, c_off[j], cs + (kCLoads * wave + j) * 1024);
#pragma unroll
        for (int j = 0; j < kWLoads; ++j) dma16(wb, w_off[j], ws + (kWLoads * wave + j) * 1024);
    };

    // ---- fragment addressing ----
    // B (c_kv^T) fragment of token block tb, k-step ks: token row
    // 128 wt + 32 tb + l32, chunk 2 ks + g.
    int b_off[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int row = 128 * wt + l32;   // + 32 tb: (row >> 2) & 3 unchanged
        b_off[ks] = row * (kKC * 2) + cslot(row, 2 * ks + g) * 16;
    }
    // A (W^T) fragment of dim block nb, k-step ks: two transposing reads.
    // Lane (g, h = bit 4, r = bits 2-3, q = bits 0-1) supplies latent row
    // 16 ks + 8 g + 4 t + r, dims 128 wn + 32 nb + 16 h + 4 q .. +4, and
    // lane 16 h + j of each half receives dim 32 nb + 16 h + j with k-slots
    // 8 g .. 8 g + 7 in natural latent order (as the c_kv fragments). The
    // swizzle depends on row % 4 = r only, so (ks, t) are immediates.
    int a_off[4];
    {
        const int tr_h = (lane >> 4) & 1;
        const int tr_r = (lane & 15) >> 2;
        const int tr_q = lane & 3;
        const int row = 8 * g + tr_r;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int chunk = (128 * wn + 32 * nb + 16 * tr_h + 4 * tr_q) / 8;
            a_off[nb] = kCBytes + row * (kNT * 2) + wslot(row, chunk) * 16 + (tr_q & 1) * 8;
        }
    }
    auto afrag = [&](const uint8_t* st, int nb, int ks) {
        bf16x8_t a;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t* p = st + a_off[nb] + (16 * ks + 4 * t) * (kNT * 2);
            const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
            const bf16x4_t y = __builtin_bit_cast(bf16x4_t, x);
            a[4 * t + 0] = y[0];
            a[4 * t + 1] = y[1];
            a[4 * t + 2] = y[2];
            a[4 * t + 3] = y[3];
        }
        return a;
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x16_t{};

    for (int s = 0; s < 3; ++s) issue(s);
    for (int s = 0; s < kSlices; ++s) {
        // slices issued: 0 .. min(s+2, last); slice s must be complete
        if (s + 2 < kSlices) wait_vmcnt<2 * kLoadsPerSlice>();
        else if (s + 1 < kSlices) wait_vmcnt<kLoadsPerSlice>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (s + 3 < kSlices) issue(s + 3);   // into slice s-1's stage, retired by the barrier
        if (wave_active) {
            const uint8_t* st = smem + (s % kStages) * kStage;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8_t a[4], b[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) a[nb] = afrag(st, nb, ks);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    b[tb] = *reinterpret_cast<const bf16x8_t*>(st + b_off[ks] + 32 * tb * (kKC * 2));
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[nb], b[tb], acc[nb][tb], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: lane owns token 128 wt + 32 tb + l32, dims in runs of 4 ----
    const int out_dim = is_v ? kDvo : kDqk;
    uint16_t* dst_base = is_v ? v_out : k_out;
    if (wave_active) {
        const int head = head0 + wn;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int t = t0 + 128 * wt + 32 * tb + l32;
            if (t < num_tokens) {
                uint16_t* dst = dst_base + ((int64_t)t * H + head) * out_dim;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
                    for (int grp = 0; grp < 4; ++grp) {
                        const int n = 32 * nb + 8 * grp + 4 * g;
                        bf16x4_t o4;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)acc[nb][tb][4 * grp + e];
                        *reinterpret_cast<bf16x4_t*>(dst + n) = o4;
                    }
                }
            }
        }
    }
    // K workgroups also place k_rope after the NoPE part of both heads
    if (!is_v) {
        constexpr int kChunksPerTok = kDrope * 2 / 16;   // 8
        for (int u = tid; u < kTT * kChunksPerTok; u += kThreads) {
            const int row = u / kChunksPerTok;
            const int c = u % kChunksPerTok;
            const int t = t0 + row;
            if (t >= num_tokens) continue;
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(k_rope + (int64_t)t * kDrope + c * 8);
            for (int hh = 0; hh < n_heads; ++hh)
                *reinterpret_cast<u32x4_t*>(k_out + ((int64_t)t * H + head0 + hh) * kDqk + kDnope + c * 8) = x;
        }
    }
}

}  // namespace

hipError_t launch_decompress(const void* c_kv, const void* k_rope, const void* w_uk,
                             const void* w_uv, int64_t num_tokens, int num_heads, void* k_out,
                             void* v_out, hipStream_t stream) {
    if (num_tokens <= 0) return hipSuccess;
    const int64_t tiles = (num_tokens + kTT - 1) / kTT;
    const int pairs = (num_heads + kHeads - 1) / kHeads;
    if (tiles > 0x7fffffff || num_heads > 65535 || num_tokens > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decompress_kernel, dim3((unsigned)tiles, (unsigned)pairs, 2),
                       dim3(kThreads), 0, stream, static_cast<const uint16_t*>(c_kv),
                       static_cast<const uint16_t*>(k_rope), static_cast<const uint16_t*>(w_uk),
                       static_cast<const uint16_t*>(w_uv), (int)num_tokens, num_heads,
                       static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
    return hipGetLastError();
}

}  // namespace mla
