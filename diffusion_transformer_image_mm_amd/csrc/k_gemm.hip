// MFMA GEMM with fused epilogues: out = epi(A W^T), fp32 accumulation.
//
// The projections of the block (QKV, output, MLP in/out; linear1/linear2 of
// the single-stream block) are dense contractions: the Luminal blog ("The
// AMD MI300X pipeline") runs them as bf16 GEMMs accumulating in fp32 with
// fused bias epilogues; here the epilogue also carries GELU, the gated
// residual add and the Euler update. Int8 weight-only layers
// (flux-amd-rocm benchmarks page) keep int8 codes in HBM and apply the
// per-channel scale to the fp32 sum.
//
// Operand formats: the weights are bf16, fp16 or int8 codes in HBM and LDS;
// bf16 and int8 weight fragments are converted in registers to fp16, which
// is exact (bf16's 8-bit significand fits fp16's 11 bits; int8 codes are
// small integers) for every weight of magnitude >= 2^-14 (smaller ones round
// at 2^-24). fp16 weights (bf16 weights converted once, the same rounding)
// skip that conversion: 12 VALU operations per 8 weights per use. The
// activation operand A (LayerNorm outputs, attention output, GELU hidden) is
// stored in fp16 by the kernel that produced it: at FLUX size, bf16 storage
// of these activations alone puts the block output at ~2e-2 of its RMS away
// from the exact result, fp16 storage at ~4e-3. The fp16 and bf16 MFMA
// rates are equal on gfx950. fp8 (OCP e4m3) operands take both A and W as
// codes with an fp32 scale per row of each, 128 k per LDS stage, on
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales; the two row
// scales multiply the fp32 sum in the epilogue.
//
// Shape of the kernels (gfx950, 64-wide wavefronts):
// * workgroup tile 256 (rows of A) x 256 (rows of W) x 64 (k);
// * fp16 and int8 weights (the block's projections) and fp8 A and W:
//   gemm_kernel4, 4 wavefronts (one per SIMD) in a 2 x 2 arrangement, each
//   owning a 128 x 128
//   sub-tile = 8 x 8 MFMA tiles of v_mfma_f32_16x16x32_f16 (or of the scaled
//   fp8 16x16x128 MFMA; 256 fp32 accumulators per lane, in AGPRs). Per MFMA this reads a third fewer operand bytes from LDS than
//   128 x 64 sub-tiles. With one wavefront per SIMD nothing hides a stalled
//   issue slot, so the main loop is laid out by hand (see there). Against the
//   eight-wavefront kernel: FLUX double block -3%, single block -2%, each
//   projection 7-10% faster alone; int8 codes are converted to fp16 in
//   small pieces between the MFMAs (FLUX-sized int8 projections 8-11% slower
//   than fp16 ones alone, against 12-16% with whole-fragment conversions;
//   the eight-wavefront kernel left the int8 denoise step 6.8% behind the
//   fp16 one);
// * bf16 and fp8-decoded weights: gemm_kernel, 8 wavefronts (two per SIMD) in a
//   2 (m) x 4 (n) arrangement, each owning a 128 x 64 sub-tile = 8 x 4 MFMA
//   tiles (128 fp32 accumulators per lane); their weight fragments are
//   converted in registers, which the second wavefront of a SIMD overlaps;
// * W is the MFMA's first operand and A the second, so the hardware result
//   is the transposed tile and each lane ends up with 4 consecutive output
//   columns of one row: 8-byte 16-bit / 16-byte fp32 epilogue stores, issued
//   row by row so that the pieces of each 128-byte output line leave back to
//   back (stored column block by column block, they left eight stores apart
//   and the output was written 1.7 times over);
// * both operand tiles go HBM/L2 -> LDS with 16-byte direct-to-LDS loads
//   (no VGPR staging), double-buffered; rows are 128 B in LDS with the
//   16-byte chunk c of row r stored at position c ^ ((r >> 1) & 7), so the
//   16 lanes that read one MFMA operand (16 rows, same chunk) hit 16
//   distinct 16-byte bank groups;
// * one barrier per k-step: in the eight-wavefront loop all fragments of
//   the current stage are read into registers before the next stage's loads
//   are issued; with fp16 weights a half-stage register pipeline instead
//   interleaves the fragment reads of one k-substep with the MFMAs of the
//   other (in its eight-wavefront form for attention-layout epilogues whose
//   head size is not a multiple of 128: a four-wavefront sub-tile spans 128
//   columns and its RMSNorm needs whole heads);
// * four-wavefront tiles stage their 16-bit and gated-residual outputs
//   through LDS and store whole rows;
// * grouped launch: up to two weight sets (text / image stream) over
//   disjoint row ranges in one grid; tiles are laid out per XCD (tile_of);
// * tail tiles: when the last round of 256-wide tiles would occupy at most
//   half of the compute units (the FLUX MLP-in projection: 864 tiles = 3
//   rounds + 96), the last row tiles run as 128-wide tiles in the same
//   launch (768 + 192 tiles: the last round becomes half as long); every
//   output element sees the same k-order either way (bit-identical);
// * head tiles: in a grouped launch the text-stream group (at most two row
//   tiles, weight slabs shared by only two tiles, so HBM-latency bound) can
//   run as 128-wide tiles dispatched first (the rule is in launch_gemm_t);
// * the epilogue of the projection that makes q, k and v (EPI_QKV_ATTN in
//   the double block; EPI_SPLIT_GELU_ATTN / EPI_SPLIT_SWIGLU_ATTN for the
//   first 3H columns of the single block's linear1) does the per-head QK
//   RMSNorm and RoPE in fp32 on the accumulators (the row's sum of squares
//   over a head: in-lane, then lanes ^16 and ^32, then the wavefronts that
//   share the head through LDS) and writes q, k and v^T straight into the
//   attention kernel's layouts, so the bf16 qkv round trip and its separate
//   kernel disappear (SGLang-AMD "Architecture Deep Dive" fuses QK
//   normalisation with RoPE; here it also joins the projection);
// * SwiGLU epilogues (a gated MLP, Luminal blog section "What the compiler
//   found on its own": the fused SwiGLU activation of Flux.2 Klein): the
//   weight keeps its natural layout, rows [gate (M) | up (M)]. A tile covers
//   128 features: tile row r loads gate row f or up row M + f of feature
//   f = 32 * (r / 64) + r % 32 (up when bit 5 of r is set), so each wavefront
//   holds gate and up of the same 32 features and the epilogue pairs its
//   accumulators in registers;
// * M and N tails: loads clamp to the last valid row, stores are guarded;
// * deterministic (no atomics, fixed k order).
#include <atomic>
#include <type_traits>

#include "common.h"

namespace mmdit {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;   // BN: the full tile; tail tiles are BN / 2 wide
constexpr int NTHREADS = 512;
constexpr int A_TILE_BYTES = BM * BK * 2;   // 32 KB
constexpr int W_TILE_BYTES_BF16 = BN * BK * 2;  // 32 KB
constexpr int W_TILE_BYTES_I8 = BN * BK;        // 16 KB

typedef __attribute__((address_space(3))) void lds_void;

MMDIT_DEV void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// f(integral_constant<int, I>) for I = B .. E-1 in order, as straight-line
// code: every index the body derives from I is a constant expression.
template <int B, int E, class F>
MMDIT_DEV void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// 16-byte direct global -> LDS load: lane i of the wavefront writes
// lds_base + 16 * i.
MMDIT_DEV void g2l_16(const void* gsrc, lds_void* lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, lds_base, 16, 0, 0);
}

// The same load written out as an instruction. The compiler does not see this
// LDS write, so its wait insertion keeps exact lgkmcnt counts for the
// fragment reads that follow (with the builtin it waits for all of them
// before the first MFMA); the caller orders the LDS accesses itself with
// s_waitcnt and barriers.
MMDIT_DEV void g2l_16_asm(const void* gsrc, uint32_t lds_addr) {
    const uint32_t l = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(gsrc) : "memory", "m0");
}
MMDIT_DEV void g2l_16_asm(const void* gsrc, lds_void* lds_base) {
    g2l_16_asm(gsrc, (uint32_t)(uintptr_t)lds_base);
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the instruction's scalar-base form: no 64-bit address
// arithmetic per lane).
MMDIT_DEV void g2l_16_asm(const char* sbase, uint32_t voff, uint32_t lds_addr) {
    const uint32_t l = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// Read an activation fragment (8 fp16) from LDS.
MMDIT_DEV f16x8_t lds_frag_h(const char* p) { return *reinterpret_cast<const f16x8_t*>(p); }

// 8 bf16 weights (one 16-byte LDS read) -> 8 fp16, pairwise.
MMDIT_DEV f16x8_t bf16x8_to_f16x8(uint4 v) {
    f16x8_t r;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = static_cast<_Float16>(__uint_as_float(w[i] << 16));
        r[2 * i + 1] = static_cast<_Float16>(__uint_as_float(w[i] & 0xffff0000u));
    }
    return r;
}

// 8 int8 codes -> 8 fp16 (exact) with 10 VALU operations. A code x biased
// to the byte u = x + 128 (xor 0x80) and placed under the fp16 exponent
// byte 0x64 is the fp16 number 1024 + u (ten mantissa bits hold u exactly);
// one packed fp16 subtraction of 1152 then leaves x, exactly. Per dword of
// four codes: one xor, two byte permutes, two packed subtractions (the
// conversion through fp32 took ~3 operations per code, and that VALU work
// delayed the matrix cores).
MMDIT_DEV f16x8_t i8x8_to_f16x8(uint2 raw) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const uint32_t w[2] = {raw.x ^ 0x80808080u, raw.y ^ 0x80808080u};
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    f16x8_t r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // bytes [0x64, u1, 0x64, u0] and [0x64, u3, 0x64, u2]
        const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, w[h], 0x04010400u);
        const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, w[h], 0x04030402u);
        const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
        const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
        r[4 * h] = a[0];
        r[4 * h + 1] = a[1];
        r[4 * h + 2] = b[0];
        r[4 * h + 3] = b[1];
    }
    return r;
}

// 8 OCP e4m3 codes -> 8 fp16 (exact: every e4m3 value is an fp16 value), two
// codes per conversion instruction through fp32.
MMDIT_DEV f16x8_t fp8x8_to_f16x8(uint2 raw) {
    f16x8_t r;
    const uint32_t w[2] = {raw.x, raw.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], true);
        r[4 * h] = static_cast<_Float16>(lo[0]);
        r[4 * h + 1] = static_cast<_Float16>(lo[1]);
        r[4 * h + 2] = static_cast<_Float16>(hi[0]);
        r[4 * h + 3] = static_cast<_Float16>(hi[1]);
    }
    return r;
}

struct TileCoord {
    int g;       // group
    int m0;      // first row of the tile within the group
    int n0;      // first output column
};

// Workgroup -> output tile. Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup b runs on XCD b % 8) and each XCD has its own L2, so each
// XCD is given one contiguous run of a tile order in which such runs are
// compact rectangles: the tile grid (the row tiles of both groups stacked,
// text rows first) is cut into CS column strips (8, 4 or 2 when the column
// count divides evenly, else 1), each strip walked in bands of RASTER_ROWS
// tile rows, column by column. An XCD then holds e.g. all 18 row tiles x 6
// columns of the MLP-in projection, or 9 rows x 9 columns of QKV, and its
// ~32 concurrent tiles share A and W rows in its L2. Both weight groups share
// the strips, so no XCD streams a whole text-stream weight matrix alone.
constexpr int RASTER_ROWS = 6;

// The grid covers row tiles [rt0, rt0 + tmt) of the stacked list.
MMDIT_DEV TileCoord tile_of(const GemmArgs& a, int bid, int total, int bn, int rt0, int tmt) {
    const int x = bid & 7, j = bid >> 3, q = total >> 3, r = total & 7;
    const int idx = x * q + (x < r ? x : r) + j;   // a bijection on [0, total)
    const int tn = (a.n + bn - 1) / bn;
    const int tm0 = (a.g[0].m + BM - 1) / BM;
    const int cs = (tn % 8 == 0) ? 8 : (tn % 4 == 0) ? 4 : (tn % 2 == 0) ? 2 : 1;
    const int cols = tn / cs;
    const int strip = idx / (tmt * cols), in_strip = idx - strip * tmt * cols;
    const int band = in_strip / (RASTER_ROWS * cols), rem = in_strip - band * RASTER_ROWS * cols;
    const int r0 = band * RASTER_ROWS;
    const int rows = (tmt - r0) < RASTER_ROWS ? (tmt - r0) : RASTER_ROWS;
    int mt = rt0 + r0 + rem % rows;
    TileCoord c;
    c.n0 = (strip * cols + rem / rows) * bn;
    if (a.ngroups == 1 || mt < tm0) {
        c.g = 0;
    } else {
        c.g = 1;
        mt -= tm0;
    }
    c.m0 = mt * BM;
    return c;
}

// Weight row loaded into tile row position v = n0 + r (a column of the
// product's output). Plain epilogues: row v. SwiGLU columns (v >= swiglu_from,
// a multiple of 256): 128 features per tile, gate and up rows interleaved in
// runs of 32 (see the header).
MMDIT_DEV int weight_row(int v, int swiglu_from, int half) {
    if (v < swiglu_from) return v;
    const int u = v - swiglu_from;
    const int f = ((u >> 6) << 5) + (u & 31);
    return swiglu_from + ((u & 32) ? half : 0) + f;
}

}  // namespace

// One output tile. TNW: MFMA sub-tiles per wavefront along n, 4 (the
// 256-wide tile) or 2 (a 128-wide tail tile). The grid's tiles of this width
// are numbered bid in [0, total) over row tiles [rt0, rt0 + tmt).
template <int WT, int EPI_T, int PIPE, int TNW>
MMDIT_DEV void gemm_tile(const GemmArgs& args, char* smem, int bid, int total, int rt0, int tmt) {
    constexpr int EPI = epi_base(EPI_T);   // the epilogue outside the attention columns
    constexpr bool INT8 = WT == MMDIT_INT8;
    constexpr bool F16W = WT == MMDIT_F16;
    constexpr bool FP8 = WT == MMDIT_FP8;      // fp8 A and W, 128 k per stage
    constexpr bool FP8W = WT == WT_FP8_W16A;   // fp8 W decoded to fp16 against fp16 A
    constexpr bool W8 = INT8 || FP8W;          // one-byte weights in the int8 LDS layout
    constexpr bool SWIGLU = EPI == MMDIT_EPI_SWIGLU || EPI == MMDIT_EPI_SPLIT_SWIGLU;
    static_assert(PIPE == 0 || F16W || (PIPE == 2 && (FP8 || INT8)), "the pipelined main loops read plain fp16, fp8 or int8 fragments");
    static_assert(TNW == 4 || (TNW == 2 && PIPE != 1 && !SWIGLU), "tail tiles: plain or 4-wavefront loop, no SwiGLU");
    static_assert(!FP8 || (TNW == 4 && !SWIGLU), "fp8: 256-wide tiles, no SwiGLU epilogue");
    constexpr int ES = FP8 ? 1 : 2;            // bytes per element of A (and of 16-bit / fp8 W)
    constexpr int BNT = 64 * TNW;                                 // tile width (output columns)
    constexpr int W_TILE = BNT * BK * (W8 ? 1 : 2);               // fp16 weights: as bf16
    constexpr int STAGE = A_TILE_BYTES + W_TILE;
    // PIPE 2: four wavefronts (one per SIMD) in a 2 x 2 arrangement, each
    // 128 x 16*TN; otherwise eight (two per SIMD) in 2 x 4
    constexpr bool W4 = PIPE == 2;
    constexpr int NWV = W4 ? 4 : 8, NWN = NWV / 2;   // wavefronts, and along n
    constexpr int TM = 8, TN = W4 ? 2 * TNW : TNW;  // MFMA sub-tiles per wavefront (m, n)
    constexpr int LA = 32 / NWV;                     // A loads per wavefront per stage
    constexpr int WL = 8 * TNW / NWV, WL8 = 4 * TNW / NWV;   // W loads per wavefront per stage (16-bit, int8)
    // stage s: A tile at smem + s*STAGE, W tile right after it

    const TileCoord tc = tile_of(args, bid, total, BNT, rt0, tmt);
    const GemmGroup& G = args.g[tc.g];
    const int M = G.m, N = args.n, K = args.k;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    // SwiGLU columns start at sw_from (0, or split_n for the split epilogue);
    // sw_half = M, the number of features
    const int sw_from = EPI == MMDIT_EPI_SPLIT_SWIGLU ? args.split_n : 0;
    const int sw_half = (N - sw_from) >> 1;

    // ---- load descriptors: a wave-uniform 64-bit base at the tile's first
    // row plus a 32-bit per-lane byte offset within the tile (so the loads
    // use the scalar-base addressing form, and the offsets span at most 256
    // rows whatever the matrix size). A tile: 256 rows x 8 chunks; wavefront
    // w issues loads j = 0..LA-1 of 8 rows each: lane i covers row
    // r = (LA w + j)*8 + i/8 at LDS position p = i%8, fetching chunk
    // c = p ^ ((r >> 1) & 7).
    const int lrow = lane >> 3, lpos = lane & 7;
    const char* a_g = reinterpret_cast<const char*>(args.a) + ((size_t)G.row0 + tc.m0) * args.lda * ES;
    uint32_t a_off_g[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int r = (wave * LA + j) * 8 + lrow;
        const int c = lpos ^ ((r >> 1) & 7);
        int gr = tc.m0 + r;
        gr = gr < M ? gr : M - 1;
        a_off_g[j] = (uint32_t)(gr - tc.m0) * (uint32_t)args.lda * (uint32_t)ES + (uint32_t)c * 16u;
    }
    // W tile. bf16: same pattern as A over N rows. int8: 64 B per row = 4
    // units of 16 codes; a load covers 16 rows (lane i: row (2w + j)*16 +
    // i/4, position i%4); unit u of row r is stored at position u ^ ((r >> 2) & 3).
    // The base row is the tile's first weight row (for SwiGLU columns the
    // first gate row; its up rows lie sw_half rows further).
    const int w_row0 = (SWIGLU && tc.n0 >= sw_from) ? sw_from + ((tc.n0 - sw_from) >> 1) : tc.n0;
    const char* w_g = static_cast<const char*>(G.w) + (size_t)w_row0 * K * (W8 ? 1 : ES);
    uint32_t w_off_g[WL];
    if (!W8) {
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const int r = (wave * WL + j) * 8 + lrow;
            const int c = lpos ^ ((r >> 1) & 7);
            int gn = tc.n0 + r;
            gn = gn < N ? gn : N - 1;
            if (SWIGLU) gn = weight_row(gn, sw_from, sw_half);
            w_off_g[j] = (uint32_t)(gn - w_row0) * (uint32_t)K * (uint32_t)ES + (uint32_t)c * 16u;
        }
    } else {
#pragma unroll
        for (int j = 0; j < WL8; ++j) {
            const int r = (wave * WL8 + j) * 16 + (lane >> 2);
            const int u = (lane & 3) ^ ((r >> 2) & 3);
            int gn = tc.n0 + r;
            gn = gn < N ? gn : N - 1;
            if (SWIGLU) gn = weight_row(gn, sw_from, sw_half);
            w_off_g[j] = (uint32_t)(gn - w_row0) * (uint32_t)K + (uint32_t)u * 16u;
        }
    }

    // LDS addresses as 32-bit offsets from the stage base (converting the
    // generic shared pointer per load cost a 64-bit round trip and a null
    // check per instruction)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto issue_stage = [&](int kt, int s) {
        const uint32_t base = lds0 + (uint32_t)(s * STAGE);
        const uint32_t ka = (uint32_t)kt * (BK * 2);
        // (the loops order their LDS accesses themselves: a wait for every
        // load and a barrier before a stage is read, so the compiler need
        // not see these writes)
        auto dma = [&](const char* g, uint32_t off, uint32_t l) { g2l_16_asm(g, off, l); };
#pragma unroll
        for (int j = 0; j < LA; ++j)
            dma(a_g, a_off_g[j] + ka, base + (uint32_t)(((wave_s * LA + j) * 8) * 128));
        const uint32_t wb = base + A_TILE_BYTES;
        if (!W8) {
#pragma unroll
            for (int j = 0; j < WL; ++j)
                dma(w_g, w_off_g[j] + ka, wb + (uint32_t)(((wave_s * WL + j) * 8) * 128));
        } else {
            const uint32_t kw = (uint32_t)kt * BK;
#pragma unroll
            for (int j = 0; j < WL8; ++j)
                dma(w_g, w_off_g[j] + kw, wb + (uint32_t)(((wave_s * WL8 + j) * 16) * 64));
        }
    };

    // ---- per-lane fragment offsets. Operand rows: lane & 15; k chunk:
    // ks*4 + (lane >> 4) for k-substep ks of the 64-wide stage.
    const int lr = lane & 15, lg = lane >> 4;
    int a_off[2], w_off[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int c = ks * 4 + lg;
        a_off[ks] = (wm * 128 + lr) * 128 + ((c ^ ((lr >> 1) & 7)) * 16);
        if (!W8)
            w_off[ks] = (wn * 16 * TN + lr) * 128 + ((c ^ ((lr >> 1) & 7)) * 16);
        else
            w_off[ks] = (wn * 16 * TN + lr) * 64 + (((c >> 1) ^ ((lr >> 2) & 3)) * 16) + (c & 1) * 8;
    }

    f32x4_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = FP8 ? K / 128 : K / BK;   // a stage holds 128 bytes of every row
    issue_stage(0, 0);
    wait_vmcnt0();
    __syncthreads();

    if constexpr (W4 && FP8) {
        // fp8 A and W, four wavefronts: a stage (128 k) is one k-step of
        // v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales), so the
        // half-stages split the columns instead: the first runs column blocks
        // 0 .. TN/2-1 and reads the other half's W fragments, the second (after
        // the barrier) runs TN/2 .. TN-1 while reading the next stage's A
        // fragments (double-buffered) and first-half W fragments and issuing
        // the next-but-one stage's direct-to-LDS loads. The MFMAs are
        // instructions tied to AGPR accumulators, in order (see the fp16 loop).
        constexpr int TH = TN / 2;   // column blocks per half-stage
        constexpr int NM = TH * TM;  // MFMAs per half-stage
        constexpr int ND = LA + WL;  // direct-to-LDS loads per stage
        constexpr int LEAD = 2;
        const int s127 = 127;        // e8m0 unit block scale
        int a_off8[2], w_off8[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = 2 * lg + h;
            a_off8[h] = (wm * 128 + lr) * 128 + ((c ^ ((lr >> 1) & 7)) * 16);
            w_off8[h] = (wn * 16 * TN + lr) * 128 + ((c ^ ((lr >> 1) & 7)) * 16);
        }
        i32x8_t fa[2][TM], fw0[TH], fw1[TH];
        auto frag8 = [&](const char* p0, const char* p1) __attribute__((always_inline)) {
            const uint4 lo = *reinterpret_cast<const uint4*>(p0);
            const uint4 hi = *reinterpret_cast<const uint4*>(p1);
            return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        auto rd_a = [&](int kt, i32x8_t* fa_, int im) __attribute__((always_inline)) {
            const char* sa = smem + (kt & 1) * STAGE;
            fa_[im] = frag8(sa + a_off8[0] + im * 16 * 128, sa + a_off8[1] + im * 16 * 128);
        };
        auto rd_w = [&](int kt, i32x8_t* fw_, int half, int j) __attribute__((always_inline)) {
            const char* sw = smem + (kt & 1) * STAGE + A_TILE_BYTES;
            const int in = half * TH + j;
            fw_[j] = frag8(sw + w_off8[0] + in * 16 * 128, sw + w_off8[1] + in * 16 * 128);
        };
        auto dma_j = [&](int kt, int s, int j) __attribute__((always_inline)) {   // load j of stage kt into buffer s
            const uint32_t base = lds0 + (uint32_t)(s * STAGE);
            const size_t ka = (size_t)kt * (BK * 2);
            if (j < LA)
                g2l_16_asm(a_g + ka, a_off_g[j], base + (uint32_t)(((wave_s * LA + j) * 8) * 128));
            else
                g2l_16_asm(w_g + ka, w_off_g[j - LA],
                           base + A_TILE_BYTES + (uint32_t)(((wave_s * WL + j - LA) * 8) * 128));
        };
        auto mf8 = [&](f32x4_t& c, const i32x8_t& w, const i32x8_t& a) __attribute__((always_inline)) {
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                         : "+a"(c)
                         : "v"(w), "v"(a), "v"(s127)
                         : "memory");
        };
        issue_stage(nk > 1 ? 1 : 0, 1);
#pragma unroll
        for (int im = 0; im < TM; ++im) rd_a(0, fa[0], im);
#pragma unroll
        for (int j = 0; j < TH; ++j) rd_w(0, fw0, 0, j);
        for (int kt = 0; kt < nk; kt += 2) {
            // two stages per trip so that the A fragment buffers have fixed names
            static_for<0, 2>([&](auto PP) __attribute__((always_inline)) {
                constexpr int par = decltype(PP)::value;   // stage kt + par uses fa[par]
                const int ks = kt + par;
                if (par == 1 && ks >= nk) return;
                // first half: column blocks 0 .. TH-1, reads of the second half's W
                static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
                    constexpr int i = decltype(I)::value;
                    mf8(acc[i / TM][i % TM], fw0[i / TM], fa[par][i % TM]);
                    if constexpr (i == LEAD - 1) __builtin_amdgcn_s_waitcnt(0xC07F);
                    static_for<0, TH>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = decltype(J)::value;
                        if constexpr (i == LEAD + ((NM - LEAD) * j) / TH) rd_w(ks, fw1, 1, j);
                    });
                });
                __builtin_amdgcn_s_waitcnt(0xC07F);
                wait_vmcnt0();
                __syncthreads();
                const int kn = ks + 2 < nk ? ks + 2 : nk - 1;
                // second half: column blocks TH .. TN-1; next stage's A and first-half W; loads of stage kn
                static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
                    constexpr int i = decltype(I)::value;
                    mf8(acc[TH + i / TM][i % TM], fw1[i / TM], fa[par][i % TM]);
                    static_for<0, TM>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = decltype(J)::value;
                        if constexpr (i == (NM * j) / (TM + TH)) rd_a(ks + 1, fa[par ^ 1], j);
                    });
                    static_for<0, TH>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = decltype(J)::value;
                        if constexpr (i == (NM * (TM + j)) / (TM + TH)) rd_w(ks + 1, fw0, 0, j);
                    });
                    static_for<0, ND>([&](auto J) __attribute__((always_inline)) {
                        constexpr int j = decltype(J)::value;
                        if constexpr (i == (NM * j) / ND) dma_j(kn, ks & 1, j);
                    });
                });
            });
        }
        wait_vmcnt0();
        asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    } else
    if constexpr (W4 && INT8) {
        // int8 weights, four wavefronts: the fp16 loop's schedule (below) with
        // each W fragment read as its 8 codes (one 8-byte LDS read) and turned
        // into fp16 as i8x8_to_f16x8 does (per 4 codes: one xor, two byte
        // permutes, two packed fp16 subtractions). An MFMA here issues every
        // 16 cycles, so the 10 instructions of a fragment are cut into six
        // parts of at most two, each placed after its own MFMA (empty asm
        // statements on a part's inputs and outputs keep it there): fragment
        // n + 1 of a half-stage after MFMAs 8n .. 8n + 5, and fragment 0 of
        // the next half-stage (read earlier in this one) after MFMAs 56 .. 61.
        // The two halves convert into separate registers, so no VALU write
        // follows an MFMA's read of the same register closely.
        static_assert(TM == 8, "six conversion parts per group of TM MFMAs");
        constexpr int NM = TN * TM;   // MFMAs per half-stage
        constexpr int NR = TN + TM;   // fragment reads per half-stage
        constexpr int ND = LA + WL8;  // direct-to-LDS loads per stage
        constexpr int LEAD = 4;
        f16x8_t r0a[TM], r1a[TM];
        uint2 r0w[TN], r1w[TN];       // codes
        uint4 c0w[TN], c1w[TN];       // fp16 fragments of the first / second half
        uint32_t t_w[2], t_lo[2], t_hi[2];   // a conversion's temporaries, per dword
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        auto rd = [&](int kt, int ks, f16x8_t* fa, uint2* fw, int j) __attribute__((always_inline)) {
            const char* sa = smem + (kt & 1) * STAGE;
            if (j < TM)
                fa[j] = lds_frag_h(sa + a_off[ks] + j * 16 * 128);
            else
                fw[j - TM] = *reinterpret_cast<const uint2*>(sa + A_TILE_BYTES + w_off[ks] + (j - TM) * 16 * 64);
        };
        auto dma_j = [&](int kt, int s, int j) __attribute__((always_inline)) {   // load j of stage kt into buffer s
            const uint32_t base = lds0 + (uint32_t)(s * STAGE);
            if (j < LA)
                g2l_16_asm(a_g + (size_t)kt * (BK * 2), a_off_g[j], base + (uint32_t)(((wave_s * LA + j) * 8) * 128));
            else
                g2l_16_asm(w_g + (size_t)kt * BK, w_off_g[j - LA],
                           base + A_TILE_BYTES + (uint32_t)(((wave_s * WL8 + j - LA) * 16) * 64));
        };
        // part q (0..5) of converting codes raw into out: dword h = q & 1,
        // step q >> 1
        auto cvt_part = [&](const uint2& raw, uint4& out, int q) __attribute__((always_inline)) {
            const int h = q & 1, st = q >> 1;
            const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
            if (st == 0) {
                uint32_t x = h ? raw.y : raw.x;
                asm volatile("" : "+v"(x));
                t_w[h] = x ^ 0x80808080u;
                t_lo[h] = __builtin_amdgcn_perm(0x64646464u, t_w[h], 0x04010400u);
                asm volatile("" : "+v"(t_w[h]), "+v"(t_lo[h]));
            } else if (st == 1) {
                t_hi[h] = __builtin_amdgcn_perm(0x64646464u, t_w[h], 0x04030402u);
                uint32_t o = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, t_lo[h]) - bias);
                asm volatile("" : "+v"(t_hi[h]), "+v"(o));
                if (h) out.z = o; else out.x = o;
            } else {
                uint32_t o = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, t_hi[h]) - bias);
                asm volatile("" : "+v"(o));
                if (h) out.w = o; else out.y = o;
            }
        };
        // one half-stage: MFMAs on (fa, cw), conversions of fw[1..] into cw
        // and of nfw[0] into ncw[0], the extra work xtra(i) after MFMA i
        auto half = [&](const f16x8_t* fa, const uint2* fw, uint4* cw, const uint2* nfw, uint4* ncw,
                        auto&& xtra) __attribute__((always_inline)) {
            static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                             : "+a"(acc[i / TM][i % TM])
                             : "v"(__builtin_bit_cast(f16x8_t, cw[i / TM])), "v"(fa[i % TM])
                             : "memory");
                xtra(I);
                if constexpr (i % TM < 6) {
                    if constexpr (i / TM + 1 < TN)
                        cvt_part(fw[i / TM + 1], cw[i / TM + 1], i % TM);
                    else
                        cvt_part(nfw[0], ncw[0], i % TM);
                }
            });
        };
        auto cvt_all = [&](const uint2& raw, uint4& out) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < 6; ++q) cvt_part(raw, out, q);
        };
        issue_stage(nk > 1 ? 1 : 0, 1);
#pragma unroll
        for (int j = 0; j < NR; ++j) rd(0, 0, r0a, r0w, j);
        cvt_all(r0w[0], c0w[0]);
        asm volatile("s_nop 4" ::: "memory");
        for (int kt = 0; kt < nk; ++kt) {
            // first half: MFMAs on r0 (substep 0 of stage kt), reads of r1 (substep 1)
            half(r0a, r0w, c0w, r1w, c1w, [&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                if constexpr (i == LEAD - 1) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                static_for<0, NR>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = decltype(J)::value;
                    if constexpr (i == LEAD + ((NM - LEAD) * j) / NR) rd(kt, 1, r1a, r1w, j);
                });
            });
            __builtin_amdgcn_s_waitcnt(0xC07F);
            wait_vmcnt0();
            __syncthreads();
            const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
            // second half: MFMAs on r1, reads of r0 (stage kt + 1), loads of stage kn
            half(r1a, r1w, c1w, r0w, c0w, [&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                static_for<0, NR>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = decltype(J)::value;
                    if constexpr (i == (NM * j) / NR) rd(kt + 1, 0, r0a, r0w, j);
                });
                static_for<0, ND>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = decltype(J)::value;
                    if constexpr (i == (NM * j) / ND + 1) dma_j(kn, kt & 1, j);
                });
            });
        }
        wait_vmcnt0();
        asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    } else
    if constexpr (W4) {
        // Four wavefronts, one per SIMD, each 128 x 16 TN (TN x TM x 4
        // accumulators, in AGPRs). The MFMAs are instructions tied to their
        // accumulator registers: issued as builtins, the compiler copied the
        // 256 accumulators between AGPRs and VGPRs inside the loop. Statements
        // in asm keep their order, so the loop is laid out here: each
        // half-stage starts with LEAD MFMAs on fragments read a half earlier,
        // waits for those reads (an s_waitcnt the compiler counts, so it need
        // not track the old and the new reads together), then spreads the
        // other half's fragment reads between its MFMAs; in the second half
        // the next-but-one stage's direct-to-LDS loads go between the MFMAs
        // too. With one wavefront per SIMD nothing hides a stalled issue slot
        // (measured: ~14 cycles of MFMA issue per direct-to-LDS load), so the
        // loads take their k-advance in the scalar base, not per lane. The
        // barrier sits between the halves, as in the eight-wavefront loop.
        constexpr int NM = TN * TM;   // MFMAs per half-stage
        constexpr int NR = TN + TM;   // fragment reads per half-stage
        constexpr int ND = LA + WL;   // direct-to-LDS loads per stage
        constexpr int LEAD = 6;       // (4: MLP-in 333-338 us, 6: 328-329 us alone; other shapes equal)
        // (the schedule is generated at compile time: every accumulator index
        // and every placement below is a constant expression)
        f16x8_t r0a[TM], r0w[TN], r1a[TM], r1w[TN];
        auto rd = [&](int kt, int ks, f16x8_t* fa, f16x8_t* fw, int j) __attribute__((always_inline)) {
            const char* sa = smem + (kt & 1) * STAGE;
            if (j < TM)
                fa[j] = lds_frag_h(sa + a_off[ks] + j * 16 * 128);
            else
                fw[j - TM] = lds_frag_h(sa + A_TILE_BYTES + w_off[ks] + (j - TM) * 16 * 128);
        };
        auto dma_j = [&](int kt, int s, int j) __attribute__((always_inline)) {   // load j of stage kt into buffer s
            const uint32_t base = lds0 + (uint32_t)(s * STAGE);
            const size_t ka = (size_t)kt * (BK * 2);
            if (j < LA)
                g2l_16_asm(a_g + ka, a_off_g[j], base + (uint32_t)(((wave_s * LA + j) * 8) * 128));
            else
                g2l_16_asm(w_g + ka, w_off_g[j - LA],
                           base + A_TILE_BYTES + (uint32_t)(((wave_s * WL + j - LA) * 8) * 128));
        };
        issue_stage(nk > 1 ? 1 : 0, 1);
#pragma unroll
        for (int j = 0; j < NR; ++j) rd(0, 0, r0a, r0w, j);
        for (int kt = 0; kt < nk; ++kt) {
            // first half: MFMAs on r0 (substep 0 of stage kt), reads of r1 (substep 1)
            static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                             : "+a"(acc[i / TM][i % TM])
                             : "v"(r0w[i / TM]), "v"(r0a[i % TM])
                             : "memory");
                if constexpr (i == LEAD - 1) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): r0 was read a half-stage ago
                static_for<0, NR>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = decltype(J)::value;
                    if constexpr (i == LEAD + ((NM - LEAD) * j) / NR) rd(kt, 1, r1a, r1w, j);
                });
            });
            __builtin_amdgcn_s_waitcnt(0xC07F);
            wait_vmcnt0();
            __syncthreads();
            // branch-free: past the end the loads repeat the last stage into the
            // free buffer and the reads fetch values that are never used
            const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
            // second half: MFMAs on r1, reads of r0 (stage kt + 1), loads of stage kn
            static_for<0, NM>([&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                             : "+a"(acc[i / TM][i % TM])
                             : "v"(r1w[i / TM]), "v"(r1a[i % TM])
                             : "memory");
                static_for<0, NR>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = decltype(J)::value;
                    if constexpr (i == (NM * j) / NR) rd(kt + 1, 0, r0a, r0w, j);
                });
                static_for<0, ND>([&](auto J) __attribute__((always_inline)) {
                    constexpr int j = decltype(J)::value;
                    if constexpr (i == (NM * j) / ND + 1) dma_j(kn, kt & 1, j);
                });
            });
        }
        wait_vmcnt0();
        // the compiler does not know the statements above are MFMAs: wait out
        // their result latency before the epilogue reads the accumulators
        asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    } else
    if constexpr (FP8) {
        // fp8: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 sub-tile and
        // stage (unit block scales). Lane l takes row l%16 and k-bytes
        // 32(l/16) .. +31 of the stage: the 16-byte chunks 2(l/16) and
        // 2(l/16)+1 of its LDS row, each at its swizzled position.
        int a_off8[2], w_off8[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = 2 * lg + h;
            a_off8[h] = (wm * 128 + lr) * 128 + ((c ^ ((lr >> 1) & 7)) * 16);
            w_off8[h] = (wn * 64 + lr) * 128 + ((c ^ ((lr >> 1) & 7)) * 16);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int s = kt & 1;
            const char* sa = smem + s * STAGE;
            const char* sw = sa + A_TILE_BYTES;
            i32x8_t fa[TM], fw[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint4 lo = *reinterpret_cast<const uint4*>(sa + a_off8[0] + i * 16 * 128);
                const uint4 hi = *reinterpret_cast<const uint4*>(sa + a_off8[1] + i * 16 * 128);
                fa[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const uint4 lo = *reinterpret_cast<const uint4*>(sw + w_off8[0] + i * 16 * 128);
                const uint4 hi = *reinterpret_cast<const uint4*>(sw + w_off8[1] + i * 16 * 128);
                fw[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            if (kt + 1 < nk) issue_stage(kt + 1, s ^ 1);
#pragma unroll
            for (int in = 0; in < TN; ++in)
#pragma unroll
                for (int im = 0; im < TM; ++im)
                    acc[in][im] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw[in], fa[im], acc[in][im], 0, 0,
                                                                                    0, 127, 0, 127);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt0();
            __syncthreads();
        }
    } else
    if (PIPE) {
        // Half-stage register pipeline for long contractions: r0 holds the
        // fragments of k-substep 0, r1 those of substep 1 (the same 96
        // registers as the plain loop). While the 32 MFMAs of one half run,
        // the 12 fragment reads of the other half are issued between them
        // (two MFMAs, one read). The barrier sits between the halves: after
        // it, stage kt+1 has landed and every wave has finished reading stage
        // kt, whose buffer then receives stage kt+2.
        f16x8_t r0a[TM], r0w[TN], r1a[TM], r1w[TN];
        auto read_half = [&](int kt, int ks, f16x8_t* fa, f16x8_t* fw) {
            const char* sa = smem + (kt & 1) * STAGE;
            const char* sw = sa + A_TILE_BYTES;
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = lds_frag_h(sa + a_off[ks] + i * 16 * 128);
#pragma unroll
            for (int i = 0; i < TN; ++i) fw[i] = lds_frag_h(sw + w_off[ks] + i * 16 * 128);
        };
        auto mfma_half = [&](const f16x8_t* fa, const f16x8_t* fw) {
#pragma unroll
            for (int in = 0; in < TN; ++in)
#pragma unroll
                for (int im = 0; im < TM; ++im)
                    acc[in][im] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw[in], fa[im], acc[in][im], 0, 0, 0);
        };
        auto interleave = [&]() {
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        };
        if (nk > 1) issue_stage(1, 1);
        read_half(0, 0, r0a, r0w);
        for (int kt = 0; kt < nk; ++kt) {
            read_half(kt, 1, r1a, r1w);
            mfma_half(r0a, r0w);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            wait_vmcnt0();
            __syncthreads();
            if (kt + 2 < nk) issue_stage(kt + 2, kt & 1);
            if (kt + 1 < nk) read_half(kt + 1, 0, r0a, r0w);
            mfma_half(r1a, r1w);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
        }
    } else
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        const char* sa = smem + s * STAGE;
        const char* sw = sa + A_TILE_BYTES;
        f16x8_t fa[2][TM], fw[2][TN];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[ks][i] = lds_frag_h(sa + a_off[ks] + i * 16 * 128);
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                if (F16W)
                    fw[ks][i] = lds_frag_h(sw + w_off[ks] + i * 16 * 128);
                else if (!W8)
                    fw[ks][i] = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(sw + w_off[ks] + i * 16 * 128));
                else if (INT8)
                    fw[ks][i] = i8x8_to_f16x8(*reinterpret_cast<const uint2*>(sw + w_off[ks] + i * 16 * 64));
                else
                    fw[ks][i] = fp8x8_to_f16x8(*reinterpret_cast<const uint2*>(sw + w_off[ks] + i * 16 * 64));
            }
        }
        if (kt + 1 < nk) issue_stage(kt + 1, s ^ 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int in = 0; in < TN; ++in)
#pragma unroll
                for (int im = 0; im < TM; ++im)
                    acc[in][im] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw[ks][in], fa[ks][im],
                                                                         acc[in][im], 0, 0, 0);
        // keep the stage wait and the barrier behind the MFMAs (the compiler
        // would otherwise hoist them, serialising the loads with the math)
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt0();
        __syncthreads();
    }

    // ---- epilogue. acc[in][im] element j: output column
    // n = n0 + wn*16*TNW + in*16 + lg*4 + j, row m = m0 + wm*128 + im*16 + lr.
    const int nb = tc.n0 + wn * 16 * TN + lg * 4;
    const int mb = tc.m0 + wm * 128 + lr;
    if (SWIGLU && tc.n0 >= sw_from) {
        // in each group of four accumulator columns (64 tile columns), in = 4q,
        // 4q + 1 hold gate and 4q + 2, 4q + 3 up of the same 32 features
        // f = (n0 - sw_from) / 2 + 8 TN wn + 32 q + 16 (in & 1) + 4 lg + j:
        // out fp16 = SiLU(gate) * up
        const int fb = ((tc.n0 - sw_from) >> 1) + wn * 8 * TN + lg * 4;
        uint16_t* obase = static_cast<uint16_t*>(EPI == MMDIT_EPI_SPLIT_SWIGLU ? args.out2 : args.out);
        const int ld = EPI == MMDIT_EPI_SPLIT_SWIGLU ? args.ldo2 : args.ldo;
        const int ocol = EPI == MMDIT_EPI_SPLIT_SWIGLU ? args.out2_col : 0;
#pragma unroll
        for (int pq = 0; pq < TN / 2; ++pq) {
            const int in = (pq >> 1) * 4 + (pq & 1);
            const int f = fb + (pq >> 1) * 32 + (pq & 1) * 16;
            const int ng = sw_from + f, nu = sw_from + sw_half + f;
            const uint2 bg = *reinterpret_cast<const uint2*>(G.bias + ng);
            const uint2 bu = *reinterpret_cast<const uint2*>(G.bias + nu);
            const float b_g[4] = {bf2f(bg.x & 0xffff), bf2f(bg.x >> 16), bf2f(bg.y & 0xffff), bf2f(bg.y >> 16)};
            const float b_u[4] = {bf2f(bu.x & 0xffff), bf2f(bu.x >> 16), bf2f(bu.y & 0xffff), bf2f(bu.y >> 16)};
            float s_g[4] = {1.f, 1.f, 1.f, 1.f}, s_u[4] = {1.f, 1.f, 1.f, 1.f};
            if (INT8 || FP8W) {
                const float4 a4 = *reinterpret_cast<const float4*>(G.scale + ng);
                const float4 c4 = *reinterpret_cast<const float4*>(G.scale + nu);
                s_g[0] = a4.x; s_g[1] = a4.y; s_g[2] = a4.z; s_g[3] = a4.w;
                s_u[0] = c4.x; s_u[1] = c4.y; s_u[2] = c4.z; s_u[3] = c4.w;
            }
#pragma unroll
            for (int im = 0; im < TM; ++im) {
                const int m = mb + im * 16;
                if (m >= M) continue;
                float y[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g = acc[in][im][j] * s_g[j] + b_g[j];
                    const float u = acc[in + 2][im][j] * s_u[j] + b_u[j];
                    y[j] = silu(g) * u;
                }
                uint16_t* o = obase + (size_t)(G.row0 + m) * ld + ocol + f;
                *reinterpret_cast<uint2*>(o) = make_uint2(pack2h(y[0], y[1]), pack2h(y[2], y[3]));
            }
        }
        return;
    }
    if (EPI_T == EPI_QKV_ATTN || (EPI_T != EPI && tc.n0 < args.split_n)) {
        // Columns [q | k | v] (split_n = 3H; H a multiple of the tile width,
        // so a tile lies in one of them; the single-stream block's MLP
        // columns follow at split_n). y = acc * s + b stays in fp32 here.
        const int H = args.split_n / 3, D = args.head_dim, seg = tc.n0 / H;
#pragma unroll
        for (int in = 0; in < TN; ++in) {
            const int n = nb + in * 16;
            const uint2 braw = *reinterpret_cast<const uint2*>(G.bias + n);
            const float b[4] = {bf2f(braw.x & 0xffff), bf2f(braw.x >> 16), bf2f(braw.y & 0xffff), bf2f(braw.y >> 16)};
            float sc[4] = {1.f, 1.f, 1.f, 1.f};
            if (INT8 || FP8 || FP8W) {
                const float4 s4 = *reinterpret_cast<const float4*>(G.scale + n);
                sc[0] = s4.x; sc[1] = s4.y; sc[2] = s4.z; sc[3] = s4.w;
            }
#pragma unroll
            for (int im = 0; im < TM; ++im) {
                float sa = 1.f;
                if (FP8) {
                    const int m = mb + im * 16;
                    sa = args.a_scale[G.row0 + (m < M ? m : M - 1)];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[in][im][j] = (acc[in][im][j] * sa) * sc[j] + b[j];
            }
        }
        if (seg < 2) {
            // The tile's slice of the RoPE table (its 256 rows x D floats: cos
            // and sin of every pair) is staged in LDS once, with 16-byte
            // direct-to-LDS loads of 1 KB per wavefront instruction; chunk c of
            // row r sits at position c ^ (r & 15), so the 16 rows read together
            // hit distinct bank groups. (Read per lane from L2 instead, every
            // entry was fetched twice, once per head of the tile, and the
            // latency sat behind the reduction's barriers.) Rows past the
            // group's end load its last row. The partial sums follow the slice.
            const int RB = D * 4;                                 // bytes per table row
            const int CPR = D / 4;                                // 16-byte chunks per row
            char* srope = smem;                                   // [256][RB]
            float* red = reinterpret_cast<float*>(smem + 256 * RB);   // [4 column waves][256 rows]
            __syncthreads();                                      // the main loop's LDS reads are done
            {
                const char* rtab = reinterpret_cast<const char*>(args.rope);
                const int rpl = 1024 / RB;                        // rows per 1 KB load
                const int loads = 256 / rpl / NWV;                // per wavefront
                for (int j = 0; j < loads; ++j) {
                    const int blk = wave * loads + j;
                    const int r = blk * rpl + lane / CPR;
                    const int c = (lane % CPR) ^ (r & 15);
                    const int m = tc.m0 + r;
                    const size_t t = (size_t)(G.row0 + (m < M ? m : M - 1));
                    g2l_16_asm(rtab + t * RB + c * 16, (lds_void*)(srope + blk * 1024));
                }
            }
            // RMSNorm over each head's D columns: lane sums over its 4 x TN
            // columns, then over the 4 lanes of its row (lane ^ 16, ^ 32), then
            // over the wavefronts that share the head, through LDS.
#pragma unroll
            for (int im = 0; im < TM; ++im) {
                float p = 0.f;
#pragma unroll
                for (int in = 0; in < TN; ++in)
#pragma unroll
                    for (int j = 0; j < 4; ++j) p += acc[in][im][j] * acc[in][im][j];
                p += __shfl_xor(p, 16, 64);
                p += __shfl_xor(p, 32, 64);
                if (lg == 0) red[wn * 256 + wm * 128 + im * 16 + lr] = p;
            }
            // fp8 operands: the exponents of q's and k's power-of-two scales,
            // from max|g| over both streams' norm scales (partial maxima of
            // the wavefronts that hold norm entries, through LDS)
            float* gpart = red + 4 * 256;            // [NWV wavefronts][2]
            if constexpr (FP8) {
                if (args.q8_out) {
                    float gq = 0.f, gk = 0.f;
                    if (tid < D) {
                        gq = fmaxf(fabsf(bf2f(args.fp8_norms[0][tid])), fabsf(bf2f(args.fp8_norms[1][tid])));
                        gk = fmaxf(fabsf(bf2f(args.fp8_norms[2][tid])), fabsf(bf2f(args.fp8_norms[3][tid])));
                    }
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) {
                        gq = fmaxf(gq, __shfl_xor(gq, o, 64));
                        gk = fmaxf(gk, __shfl_xor(gk, o, 64));
                    }
                    if (lane == 0) {
                        gpart[2 * wave] = gq;
                        gpart[2 * wave + 1] = gk;
                    }
                }
            }
            wait_vmcnt0();   // this wavefront's slice loads have landed
            __syncthreads();
            int e8 = 0;                              // this segment's exponent (fp8 operands)
            if constexpr (FP8) {
                if (args.q8_out) {
                    float gq = 0.f, gk = 0.f;
#pragma unroll
                    for (int w = 0; w < NWV; ++w) {
                        gq = fmaxf(gq, gpart[2 * w]);
                        gk = fmaxf(gk, gpart[2 * w + 1]);
                    }
                    const int eq = ceil_log2_exp(args.fp8_bound * gq), ek = ceil_log2_exp(args.fp8_bound * gk);
                    e8 = seg == 0 ? eq : ek;
                    if (tid == 0 && tc.n0 == 0) {    // every first column tile stores the same pair
                        args.fp8_exps[0] = eq;
                        args.fp8_exps[1] = ek;
                    }
                }
            }
            const int wph = D / (16 * TN);         // wavefronts per head: 1, 2 or 4 (D a multiple of 16 TN)
            const int w0 = (wn / wph) * wph;
            const uint16_t* gsc = seg == 0 ? G.qn : G.kn;
            uint16_t* dst = seg == 0 ? args.q_out : args.k_out;
            const int nsb = nb - seg * H;           // the lane's first column within q (or k)
            const int h = nsb / D;                  // every column of a wavefront is in one head
            float gs[TN][4];
#pragma unroll
            for (int in = 0; in < TN; ++in) {
                const uint2 graw = *reinterpret_cast<const uint2*>(gsc + (nsb + in * 16) % D);
                gs[in][0] = bf2f(graw.x & 0xffff); gs[in][1] = bf2f(graw.x >> 16);
                gs[in][2] = bf2f(graw.y & 0xffff); gs[in][3] = bf2f(graw.y >> 16);
            }
            const float inv_d = 1.0f / (float)D;
#pragma unroll
            for (int im = 0; im < TM; ++im) {
                const int m = mb + im * 16;
                if (m >= M) continue;
                float ss = 0.f;
                for (int w = 0; w < wph; ++w) ss += red[(w0 + w) * 256 + wm * 128 + im * 16 + lr];
                const float rstd = 1.0f / sqrtf(ss * inv_d + args.rms_eps);
                const size_t t = (size_t)(G.row0 + m);
                const int r = wm * 128 + im * 16 + lr;   // the row within the tile
#pragma unroll
                for (int in = 0; in < TN; ++in) {
                    const int dl = (nsb + in * 16) % D;   // 4 consecutive dims dl..dl+3: pairs dl/2, dl/2+1
                    const float4 c =
                        *reinterpret_cast<const float4*>(srope + r * RB + (((dl >> 2) ^ (r & 15)) << 4));
                    const float a0 = acc[in][im][0] * rstd * gs[in][0], b0 = acc[in][im][1] * rstd * gs[in][1];
                    const float a1 = acc[in][im][2] * rstd * gs[in][2], b1 = acc[in][im][3] * rstd * gs[in][3];
                    const float y0 = a0 * c.x - b0 * c.y, y1 = a0 * c.y + b0 * c.x;
                    const float y2 = a1 * c.z - b1 * c.w, y3 = a1 * c.w + b1 * c.z;
                    if (FP8 && args.q8_out) {
                        // e4m3 codes of the fp32 values at 2^e8 (the RMSNorm bound keeps
                        // them within 448; the clamp only guards the conversion)
                        auto q8 = [&](float x) { return fminf(fmaxf(ldexpf(x, -e8), -448.0f), 448.0f); };
                        uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(q8(y0), q8(y1), 0u, false);
                        pk = __builtin_amdgcn_cvt_pk_fp8_f32(q8(y2), q8(y3), pk, true);
                        uint8_t* dst8 = seg == 0 ? args.q8_out : args.k8_out;
                        *reinterpret_cast<uint32_t*>(dst8 + ((size_t)h * args.l_pad + t) * D + dl) = pk;
                    } else {
                        *reinterpret_cast<uint2*>(dst + ((size_t)h * args.l_pad + t) * D + dl) =
                            make_uint2(pack2bf(y0, y1), pack2bf(y2, y3));
                    }
                }
            }
        } else {
            // v: transposed; inside each aligned group of 16 keys the quads are
            // stored in the order 0, 2, 1, 3 (the attention kernel's operand order)
            const int nsb = nb - 2 * H;
            const int h = nsb / D;
#pragma unroll
            for (int im = 0; im < TM; ++im) {
                const int m = mb + im * 16;
                if (m >= M) continue;
                const int t = G.row0 + m;
                const int qd = (t >> 2) & 3;
                const int pos = (t & ~15) | ((((qd & 1) << 1) | (qd >> 1)) << 2) | (t & 3);
#pragma unroll
                for (int in = 0; in < TN; ++in) {
                    const int dl = (nsb + in * 16) % D;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        args.vt_out[((size_t)h * D + dl + j) * args.l_pad + pos] = f2bf(acc[in][im][j]);
                }
            }
        }
        return;
    }
    // Four-wavefront tiles stage their outputs through LDS (the stage buffers
    // are free after the main loop) and store whole rows: stored straight from
    // the MFMA layout, each instruction writes 16 rows x 32 or 64 bytes, and
    // with every tile of a round reaching its epilogue together those partial
    // lines were issued at ~7 bytes/clk per CU (measured; the whole-row stores
    // below write 2-4 full 128-byte lines per instruction). LDS row r holds
    // its 16-byte chunk q at position q ^ (r & 15): the 16 rows a store
    // instruction writes fall in distinct bank groups, and a row read is a
    // permutation within the row.
    if constexpr (W4 && (F16W || FP8 || INT8) && (EPI == MMDIT_EPI_BIAS || EPI == MMDIT_EPI_BIAS_GELU || EPI == MMDIT_EPI_SPLIT_GELU)) {
        const bool mlp = EPI == MMDIT_EPI_BIAS_GELU || (EPI == MMDIT_EPI_SPLIT_GELU && tc.n0 >= args.split_n);
        uint16_t* obase = static_cast<uint16_t*>(args.out);
        int ld = args.ldo, ocol = 0;
        if (EPI == MMDIT_EPI_SPLIT_GELU && mlp) {
            obase = static_cast<uint16_t*>(args.out2);
            ld = args.ldo2;
            ocol = args.out2_col - args.split_n;
        }
        const bool one_side = EPI != MMDIT_EPI_SPLIT_GELU || mlp || tc.n0 + BNT <= args.split_n;
        if (one_side && N % 8 == 0 && ld % 8 == 0 && ocol % 8 == 0) {
            constexpr int RWB = BNT * 2;          // bytes per staged row
            constexpr int CPR = RWB / 16;         // 16-byte chunks per row
            float bv[TN][4], scv[TN][4];
#pragma unroll
            for (int in = 0; in < TN; ++in) {
                const int n = nb + in * 16;
                const int nc = n < N ? n : N - 4;
                const uint2 braw = *reinterpret_cast<const uint2*>(G.bias + nc);
                bv[in][0] = bf2f(braw.x & 0xffff); bv[in][1] = bf2f(braw.x >> 16);
                bv[in][2] = bf2f(braw.y & 0xffff); bv[in][3] = bf2f(braw.y >> 16);
                if constexpr (FP8 || INT8) {
                    const float4 s4 = *reinterpret_cast<const float4*>(G.scale + nc);
                    scv[in][0] = s4.x; scv[in][1] = s4.y; scv[in][2] = s4.z; scv[in][3] = s4.w;
                }
            }
            __syncthreads();   // every wavefront's loads have landed and its reads are done
#pragma unroll
            for (int im = 0; im < TM; ++im) {
                const int r = wm * 128 + im * 16 + lr;
                float sa = 1.f;
                if constexpr (FP8) sa = args.a_scale[G.row0 + (mb + im * 16 < M ? mb + im * 16 : M - 1)];
#pragma unroll
                for (int in = 0; in < TN; ++in) {
                    const int q = wn * 2 * TN + in * 2 + (lg >> 1);
                    float y[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        y[j] = FP8    ? (acc[in][im][j] * sa) * scv[in][j] + bv[in][j]
                               : INT8 ? acc[in][im][j] * scv[in][j] + bv[in][j]
                                      : acc[in][im][j] + bv[in][j];
                    uint2 pk;
                    if (mlp) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) y[j] = gelu_tanh(y[j]);
                        pk = make_uint2(pack2h(y[0], y[1]), pack2h(y[2], y[3]));
                    } else {
                        pk = make_uint2(pack2bf(y[0], y[1]), pack2bf(y[2], y[3]));
                    }
                    *reinterpret_cast<uint2*>(smem + r * RWB + ((q ^ (r & 15)) << 4) + (lg & 1) * 8) = pk;
                }
            }
            __syncthreads();
#pragma unroll 4
            for (int i = 0; i < CPR; ++i) {
                const int idx = i * (NTHREADS / 2) + tid;
                const int r = idx / CPR, q = idx % CPR;
                const uint4 v = *reinterpret_cast<const uint4*>(smem + r * RWB + ((q ^ (r & 15)) << 4));
                const int m = tc.m0 + r, n = tc.n0 + q * 8;
                if (m < M && n < N)
                    *reinterpret_cast<uint4*>(obase + (size_t)(G.row0 + m) * ld + ocol + n) = v;
            }
            return;
        }
    }
    if constexpr (W4 && (F16W || FP8 || INT8) && EPI == MMDIT_EPI_GATE_RESID) {
        if (N % 4 == 0 && args.ldo % 4 == 0 && args.ldr % 4 == 0) {
            // fp32 out = resid + gate * (acc + bias) in two passes of half the
            // columns: pass p stages column blocks p TN/2 .. of every wavefront
            // (two stripes of 16 TN/2 columns per row), then the rows are read
            // back, the residual and gate applied, and stored 16 bytes per lane
            constexpr int SPW = TN / 2;           // column blocks per wavefront and pass
            constexpr int RWB = BNT * 2;          // bytes per staged row: BNT/2 fp32
            constexpr int CPR = RWB / 16;
            constexpr int CPS = SPW * 4;          // chunks per stripe
            float bv[TN][4], scv[TN][4], sav[TM];
#pragma unroll
            for (int in = 0; in < TN; ++in) {
                const int n = nb + in * 16;
                const int nc = n < N ? n : N - 4;
                const uint2 braw = *reinterpret_cast<const uint2*>(G.bias + nc);
                bv[in][0] = bf2f(braw.x & 0xffff); bv[in][1] = bf2f(braw.x >> 16);
                bv[in][2] = bf2f(braw.y & 0xffff); bv[in][3] = bf2f(braw.y >> 16);
                if constexpr (FP8 || INT8) {
                    const float4 s4 = *reinterpret_cast<const float4*>(G.scale + nc);
                    scv[in][0] = s4.x; scv[in][1] = s4.y; scv[in][2] = s4.z; scv[in][3] = s4.w;
                }
            }
            if constexpr (FP8) {
#pragma unroll
                for (int im = 0; im < TM; ++im)
                    sav[im] = args.a_scale[G.row0 + (mb + im * 16 < M ? mb + im * 16 : M - 1)];
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                __syncthreads();   // the loop's (or the previous pass's) LDS accesses are done
#pragma unroll
                for (int im = 0; im < TM; ++im) {
                    const int r = wm * 128 + im * 16 + lr;
#pragma unroll
                    for (int b = 0; b < SPW; ++b) {
                        const int in = p * SPW + b;
                        const int q = wn * CPS + b * 4 + lg;
                        float y[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            y[j] = FP8    ? (acc[in][im][j] * sav[im]) * scv[in][j] + bv[in][j]
                                   : INT8 ? acc[in][im][j] * scv[in][j] + bv[in][j]
                                          : acc[in][im][j] + bv[in][j];
                        *reinterpret_cast<float4*>(smem + r * RWB + ((q ^ (r & 15)) << 4)) =
                            make_float4(y[0], y[1], y[2], y[3]);
                    }
                }
                __syncthreads();
                // out may alias resid: a batch's residual (and gate) loads are
                // issued together, from clamped addresses, before its stores
                constexpr int BB = 8;
#pragma unroll
                for (int i0 = 0; i0 < CPR; i0 += BB) {
                    float4 rr[BB], g4[BB];
#pragma unroll
                    for (int ii = 0; ii < BB; ++ii) {
                        const int idx = (i0 + ii) * (NTHREADS / 2) + tid;
                        const int r = idx / CPR, q = idx % CPR;
                        const int m = tc.m0 + r;
                        const int n = tc.n0 + (q / CPS) * 16 * TN + p * SPW * 16 + (q % CPS) * 4;
                        const size_t grow = (size_t)(G.row0 + (m < M ? m : M - 1));
                        const int nc = n < N ? n : N - 4;
                        rr[ii] = *reinterpret_cast<const float4*>(args.resid + grow * args.ldr + nc);
                        g4[ii] = *reinterpret_cast<const float4*>(G.gate + nc);
                    }
#pragma unroll
                    for (int ii = 0; ii < BB; ++ii) {
                        const int idx = (i0 + ii) * (NTHREADS / 2) + tid;
                        const int r = idx / CPR, q = idx % CPR;
                        const int m = tc.m0 + r;
                        const int n = tc.n0 + (q / CPS) * 16 * TN + p * SPW * 16 + (q % CPS) * 4;
                        if (m < M && n < N) {
                            const float4 y = *reinterpret_cast<const float4*>(smem + r * RWB + ((q ^ (r & 15)) << 4));
                            *reinterpret_cast<float4*>(static_cast<float*>(args.out) + (size_t)(G.row0 + m) * args.ldo + n) =
                                make_float4(rr[ii].x + g4[ii].x * y.x, rr[ii].y + g4[ii].y * y.y,
                                            rr[ii].z + g4[ii].z * y.z, rr[ii].w + g4[ii].w * y.w);
                        }
                    }
                }
            }
            return;
        }
    }
    // Per-column values of the lane's 4 x TN output columns, then the rows:
    // the TN stores of one row (its 16 x TN columns, i.e. whole 128-byte lines
    // of 16-bit output) are issued back to back.
    float b[TN][4], sc[TN][4], gt[TN][4];
#pragma unroll
    for (int in = 0; in < TN; ++in) {
        const int n = nb + in * 16;
        const int nc = n < N ? n : N - 4;   // out-of-range columns: read a valid column group, store nothing
        const uint2 braw = *reinterpret_cast<const uint2*>(G.bias + nc);
        b[in][0] = bf2f(braw.x & 0xffff); b[in][1] = bf2f(braw.x >> 16);
        b[in][2] = bf2f(braw.y & 0xffff); b[in][3] = bf2f(braw.y >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) { sc[in][j] = 1.f; gt[in][j] = 0.f; }
        if (INT8 || FP8 || FP8W) {
            const float4 s4 = *reinterpret_cast<const float4*>(G.scale + nc);
            sc[in][0] = s4.x; sc[in][1] = s4.y; sc[in][2] = s4.z; sc[in][3] = s4.w;
        }
        if (EPI == MMDIT_EPI_GATE_RESID) {
            const float4 g4 = *reinterpret_cast<const float4*>(G.gate + nc);
            gt[in][0] = g4.x; gt[in][1] = g4.y; gt[in][2] = g4.z; gt[in][3] = g4.w;
        }
    }
    if constexpr (EPI == MMDIT_EPI_GATE_RESID) {
        // out = resid + gate * y, out possibly aliasing resid: the residual
        // loads of 2-4 rows are issued together (clamped addresses, so the
        // loads are straight-line and stay in bounds) before those rows are
        // stored; loaded one by one between the stores (which may alias
        // them) they were 32 serial round trips per lane
        constexpr int RB = (INT8 || FP8 || FP8W || TN > 4) ? 2 : 4;   // (those hold per-column scales or twice the columns)
#pragma unroll
        for (int i0 = 0; i0 < TM; i0 += RB) {
            float4 r[RB][TN];
#pragma unroll
            for (int ii = 0; ii < RB; ++ii) {
                const int m = mb + (i0 + ii) * 16;
                const size_t grow = (size_t)(G.row0 + (m < M ? m : M - 1));
#pragma unroll
                for (int in = 0; in < TN; ++in) {
                    const int n = nb + in * 16;
                    r[ii][in] = *reinterpret_cast<const float4*>(args.resid + grow * args.ldr + (n < N ? n : N - 4));
                }
            }
#pragma unroll
            for (int ii = 0; ii < RB; ++ii) {
                const int m = mb + (i0 + ii) * 16;
                if (m >= M) continue;
                const size_t grow = (size_t)(G.row0 + m);
                const float sa = FP8 ? args.a_scale[grow] : 1.f;
#pragma unroll
                for (int in = 0; in < TN; ++in) {
                    const int n = nb + in * 16;
                    if (n >= N) continue;
                    float y[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        y[j] = FP8 ? (acc[in][i0 + ii][j] * sa) * sc[in][j] + b[in][j]
                                   : acc[in][i0 + ii][j] * sc[in][j] + b[in][j];
                    const float4 rr = r[ii][in];
                    *reinterpret_cast<float4*>(static_cast<float*>(args.out) + grow * args.ldo + n) =
                        make_float4(rr.x + gt[in][0] * y[0], rr.y + gt[in][1] * y[1], rr.z + gt[in][2] * y[2],
                                    rr.w + gt[in][3] * y[3]);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int im = 0; im < TM; ++im) {
        const int m = mb + im * 16;
        if (m >= M) continue;
        const size_t grow = (size_t)(G.row0 + m);
        float sa = 1.f;
        if (FP8) sa = args.a_scale[grow];   // the row's activation scale
#pragma unroll
        for (int in = 0; in < TN; ++in) {
            const int n = nb + in * 16;
            if (n >= N) continue;
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                y[j] = FP8 ? (acc[in][im][j] * sa) * sc[in][j] + b[in][j] : acc[in][im][j] * sc[in][j] + b[in][j];
            if (EPI == MMDIT_EPI_BIAS || EPI == MMDIT_EPI_SPLIT_SWIGLU ||
                (EPI == MMDIT_EPI_SPLIT_GELU && n < args.split_n)) {
                // attention-side operands (q, k, v): bf16
                uint16_t* o = static_cast<uint16_t*>(args.out) + grow * args.ldo + n;
                *reinterpret_cast<uint2*>(o) = make_uint2(pack2bf(y[0], y[1]), pack2bf(y[2], y[3]));
            } else if (EPI == MMDIT_EPI_BIAS_GELU) {
                // MLP hidden, the next projection's activation operand: fp16
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = gelu_tanh(y[j]);
                uint16_t* o = static_cast<uint16_t*>(args.out) + grow * args.ldo + n;
                *reinterpret_cast<uint2*>(o) = make_uint2(pack2h(y[0], y[1]), pack2h(y[2], y[3]));
            } else if (EPI == MMDIT_EPI_SPLIT_GELU) {
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = gelu_tanh(y[j]);
                uint16_t* o = static_cast<uint16_t*>(args.out2) + grow * args.ldo2 + args.out2_col +
                              (n - args.split_n);
                *reinterpret_cast<uint2*>(o) = make_uint2(pack2h(y[0], y[1]), pack2h(y[2], y[3]));
            } else if (EPI == MMDIT_EPI_GATE_RESID) {
                const float4 r = *reinterpret_cast<const float4*>(args.resid + grow * args.ldr + n);
                float4 o4 = make_float4(r.x + gt[in][0] * y[0], r.y + gt[in][1] * y[1], r.z + gt[in][2] * y[2],
                                        r.w + gt[in][3] * y[3]);
                *reinterpret_cast<float4*>(static_cast<float*>(args.out) + grow * args.ldo + n) = o4;
            } else if (EPI == MMDIT_EPI_BIAS_F32) {
                *reinterpret_cast<float4*>(static_cast<float*>(args.out) + grow * args.ldo + n) =
                    make_float4(y[0], y[1], y[2], y[3]);
            } else if (EPI == MMDIT_EPI_EULER) {
                float* o = static_cast<float*>(args.out) + grow * args.ldo + n;
                float4 z = *reinterpret_cast<float4*>(o);
                z.x += args.alpha * y[0]; z.y += args.alpha * y[1];
                z.z += args.alpha * y[2]; z.w += args.alpha * y[3];
                *reinterpret_cast<float4*>(o) = z;
            }
        }
    }
}

template <int WT, int EPI, int PIPE>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(const GemmArgs args) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    constexpr bool SWIGLU = epi_base(EPI) == MMDIT_EPI_SWIGLU || epi_base(EPI) == MMDIT_EPI_SPLIT_SWIGLU;
    const int tm0 = (args.g[0].m + BM - 1) / BM;
    const int tmt = args.ngroups == 2 ? tm0 + (args.g[1].m + BM - 1) / BM : tm0;
    const int nf = args.full_tiles;
    if constexpr (!SWIGLU && WT != MMDIT_FP8) {
        if (args.head_rows > 0) {
            const int nh = args.head_rows * ((args.n + BN / 2 - 1) / (BN / 2));
            if ((int)blockIdx.x < nh) {
                gemm_tile<WT, EPI, 0, 2>(args, smem, blockIdx.x, nh, 0, args.head_rows);
                return;
            }
            gemm_tile<WT, EPI, PIPE, 4>(args, smem, blockIdx.x - nh, nf, args.head_rows, tmt - args.head_rows);
            return;
        }
    }
    if constexpr (!SWIGLU && WT != MMDIT_FP8) {
        if ((int)blockIdx.x >= nf) {
            gemm_tile<WT, EPI, 0, 2>(args, smem, blockIdx.x - nf, gridDim.x - nf, tmt - args.tail_rows,
                                     args.tail_rows);
            return;
        }
    }
    gemm_tile<WT, EPI, PIPE, 4>(args, smem, blockIdx.x, nf, 0, tmt - args.tail_rows);
}

// The four-wavefront kernel (fp16 weights): the same tile dispatch as
// gemm_kernel with 256 threads per workgroup.
template <int WT, int EPI>
__global__ __launch_bounds__(NTHREADS / 2, 1) void gemm_kernel4(const GemmArgs args) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    constexpr bool SWIGLU = epi_base(EPI) == MMDIT_EPI_SWIGLU || epi_base(EPI) == MMDIT_EPI_SPLIT_SWIGLU;
    const int tm0 = (args.g[0].m + BM - 1) / BM;
    const int tmt = args.ngroups == 2 ? tm0 + (args.g[1].m + BM - 1) / BM : tm0;
    const int nf = args.full_tiles;
    if constexpr (!SWIGLU && WT != MMDIT_FP8) {
        if (args.head_rows > 0) {
            const int nh = args.head_rows * ((args.n + BN / 2 - 1) / (BN / 2));
            if ((int)blockIdx.x < nh) {
                gemm_tile<WT, EPI, 2, 2>(args, smem, blockIdx.x, nh, 0, args.head_rows);
                return;
            }
            gemm_tile<WT, EPI, 2, 4>(args, smem, blockIdx.x - nh, nf, args.head_rows, tmt - args.head_rows);
            return;
        }
        if ((int)blockIdx.x >= nf) {
            gemm_tile<WT, EPI, 2, 2>(args, smem, blockIdx.x - nf, gridDim.x - nf, tmt - args.tail_rows,
                                     args.tail_rows);
            return;
        }
    }
    gemm_tile<WT, EPI, 2, 4>(args, smem, blockIdx.x, nf, 0, tmt - args.tail_rows);
}

// Length, in half tile-times, of a launch that dispatches n_half tiles of
// half a tile-time and then n_full tiles of one tile-time, in grid order,
// each to the first compute unit that becomes free (cus units).
static int launch_half_units(int n_half, int n_full, int cus) {
    int freed[3] = {cus, 0, 0};   // units that become free at t, t + 1, t + 2
    int end = 0;
    for (int t = 0; n_half + n_full > 0; ++t) {
        int avail = freed[t % 3];
        freed[t % 3] = 0;
        const int h = avail < n_half ? avail : n_half;
        n_half -= h;
        avail -= h;
        const int f = avail < n_full ? avail : n_full;
        n_full -= f;
        freed[(t + 1) % 3] += h;
        freed[(t + 2) % 3] += f;
        if (h) end = end > t + 1 ? end : t + 1;
        if (f) end = end > t + 2 ? end : t + 2;
        freed[(t + 1) % 3] += avail - f;   // idle units stay free
    }
    return end;
}

constexpr int kMaxDevices = 64;

// Compute units of the current device. The only per-process values the
// library keeps are caches of device properties like this one, per device
// and thread-safe (a relaxed atomic: every thread that races here stores the
// same number); results never depend on them.
static int cu_count() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev < 0 || dev >= kMaxDevices) {
        int n = 0;
        return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    }
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
        c = n;
    }
    return c;
}

// Sets a kernel's dynamic-LDS limit on the current device once per device
// (the attribute is per device; setting it again is harmless, so a race only
// repeats the call). done: one bit per device of that kernel.
static hipError_t lds_attribute_once(const void* kfn, int lds, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < kMaxDevices ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// The kernel for weight type WT and epilogue E: fp16 weights take the
// four-wavefront kernel (w4) or the pipelined eight-wavefront one, the other
// formats the plain eight-wavefront loop.
template <int WT, int E>
static void (*gemm_kernel_for(bool w4))(const GemmArgs) {
    if constexpr (WT == MMDIT_F16) {
        if (w4) return gemm_kernel4<WT, E>;
        return gemm_kernel<WT, E, 1>;
    } else if constexpr (WT == MMDIT_FP8 && epi_base(E) != MMDIT_EPI_SWIGLU && epi_base(E) != MMDIT_EPI_SPLIT_SWIGLU) {
        if (w4) return gemm_kernel4<WT, E>;
        return gemm_kernel<WT, E, 0>;
    } else if constexpr (WT == MMDIT_INT8) {
        if (w4) return gemm_kernel4<WT, E>;
        return gemm_kernel<WT, E, 0>;
    } else {
        (void)w4;
        return gemm_kernel<WT, E, 0>;
    }
}

template <int WT>
static hipError_t launch_gemm_t(const GemmArgs& a0, hipStream_t s) {
    constexpr bool W8 = WT == MMDIT_INT8 || WT == WT_FP8_W16A;   // one-byte weight tiles
    GemmArgs a = a0;
    const int tn = (a.n + BN - 1) / BN;
    int tmt = 0;
    for (int g = 0; g < a.ngroups; ++g) tmt += (a.g[g].m + BM - 1) / BM;
    if (tmt == 0 || tn == 0) return hipSuccess;
    const bool swiglu = epi_base(a.epilogue) == MMDIT_EPI_SWIGLU || epi_base(a.epilogue) == MMDIT_EPI_SPLIT_SWIGLU;
    // fp16 weights take the pipelined loop at every K (measured against the
    // plain loop: +10% at K = 12288, +3% at K = 15360; at K = 3072 -1% to +1%
    // alone, and the FLUX double block 1.351 -> 1.339 ms once the tail tiles
    // (which keep the plain loop) run inside the pipelined kernels too,
    // alternating processes on one box).
    const bool pipe = WT == MMDIT_F16;
    // ... and with fp16, int8 or fp8 operands the four-wavefront kernel,
    // whose wavefronts hold 128 x 128 of the tile (a third fewer LDS fragment
    // reads per MFMA); its attention-layout epilogues need whole heads per
    // wavefront
    const bool attn_epi0 = a.epilogue == EPI_QKV_ATTN || a.epilogue == EPI_SPLIT_GELU_ATTN ||
                           a.epilogue == EPI_SPLIT_SWIGLU_ATTN;
    const bool w4 = (WT == MMDIT_F16 || WT == MMDIT_FP8 || WT == MMDIT_INT8) && (!attn_epi0 || a.head_dim % 128 == 0);
    // Tail tiles: when the last round of 256-wide tiles would fill at most
    // half of the compute units, and the last r row tiles can be cut off so
    // that the rest fills whole rounds, those r row tiles run as 128-wide
    // tiles instead (twice as many, each half as long).
    const int cus = cu_count();
    a.tail_rows = 0;
    if (WT != MMDIT_FP8 && !swiglu && (tmt * tn) % cus != 0 && (tmt * tn) % cus <= cus / 2) {
        const int tn2 = (a.n + BN / 2 - 1) / (BN / 2);
        for (int r = 1; r < tmt; ++r) {
            if (((tmt - r) * tn) % cus == 0 && r * tn2 <= cus) {
                a.tail_rows = r;
                break;
            }
        }
    }
    a.full_tiles = (tmt - a.tail_rows) * tn;
    int tiles = a.full_tiles + a.tail_rows * ((a.n + BN / 2 - 1) / (BN / 2));
    // Head tiles: in a grouped launch whose first group has at most two row
    // tiles (the text stream: 512 rows), that group can run as 128-wide tiles
    // dispatched ahead of the 256-wide ones, in place of tail tiles. Its
    // weight slabs are shared by only two tiles, so its k-steps wait on HBM,
    // not L2, and its tiles are the slowest of the launch; halved and started
    // first they no longer set its end. They are used when, counting every
    // 256-wide tile as one tile-time, the launch gets no longer than with the
    // plain (or tail-tile) dispatch: the FLUX double block's four projections
    // (216, 648, 864 tiles: ties), not Flux.2 Klein's QKV at 512x512 (480
    // tiles: 2 -> 2.5 tile-times) or its launches of whole rounds. Measured:
    // FLUX double block 1.455 -> 1.431 ms and 1.430 -> 1.408 ms (same-process
    // A/B on two boxes; a third showed no change), Klein double block at
    // 512x512 1.359 -> 1.341 ms, larger Klein blocks unchanged; outputs are
    // bit-identical (every element keeps its k-order).
    a.head_rows = 0;
    {
        const int tm0g = (a.g[0].m + BM - 1) / BM;
        const int tn2 = (a.n + BN / 2 - 1) / (BN / 2);
        const int now = a.tail_rows ? launch_half_units(0, a.full_tiles, cus) + 1
                                    : launch_half_units(0, tmt * tn, cus);
        if (WT != MMDIT_FP8 && !swiglu && a.ngroups == 2 && tm0g <= 2 && (tm0g * tn2) % 8 == 0 &&
            launch_half_units(tm0g * tn2, (tmt - tm0g) * tn, cus) <= now) {
            a.head_rows = tm0g;
            a.tail_rows = 0;
            a.full_tiles = (tmt - tm0g) * tn;
            tiles = a.full_tiles + tm0g * tn2;
        }
    }
    // the attention-layout epilogues stage a 256 x D fp32 RoPE slice (D <= 128)
    // and the RMSNorm partial sums in LDS after the main loop
    const bool attn_epi = a.epilogue == EPI_QKV_ATTN || a.epilogue == EPI_SPLIT_GELU_ATTN ||
                          a.epilogue == EPI_SPLIT_SWIGLU_ATTN;
    const size_t lds_main = 2 * (size_t)(A_TILE_BYTES + (W8 ? W_TILE_BYTES_I8 : W_TILE_BYTES_BF16));
    const size_t lds_epi = 256 * 128 * 4 + 4 * 256 * 4 + 16 * 4;   // + the fp8 exponents' partial maxima
    size_t lds = attn_epi && lds_epi > lds_main ? lds_epi : lds_main;
    // the four-wavefront tiles stage their 16-bit and gated-residual outputs
    // in LDS: 256 rows x 512 bytes (more than two int8-weight stages)
    if (w4 && lds < (size_t)256 * 512) lds = (size_t)256 * 512;
    dim3 grid(tiles), block(w4 ? NTHREADS / 2 : NTHREADS);
#define GEMM_CASE(E)                                                                        \
    case E: if constexpr (WT == MMDIT_FP8 && (epi_base(E) == MMDIT_EPI_SWIGLU || epi_base(E) == MMDIT_EPI_SPLIT_SWIGLU)) { \
        return hipErrorInvalidValue;                                                        \
    } else {                                                                                \
        auto kfn = gemm_kernel_for<WT, E>(w4);                                              \
        static std::atomic<uint64_t> attr_done[3];                                          \
        hipError_t e = lds_attribute_once((const void*)kfn, (int)lds, attr_done[w4 ? 2 : pipe]); \
        if (e != hipSuccess) return e;                                                      \
        hipLaunchKernelGGL(kfn, grid, block, lds, s, a);                                    \
        break;                                                                              \
    }
    switch (a.epilogue) {
        GEMM_CASE(MMDIT_EPI_BIAS)
        GEMM_CASE(MMDIT_EPI_BIAS_GELU)
        GEMM_CASE(MMDIT_EPI_GATE_RESID)
        GEMM_CASE(MMDIT_EPI_SPLIT_GELU)
        GEMM_CASE(MMDIT_EPI_BIAS_F32)
        GEMM_CASE(MMDIT_EPI_EULER)
        GEMM_CASE(MMDIT_EPI_SWIGLU)
        GEMM_CASE(MMDIT_EPI_SPLIT_SWIGLU)
        GEMM_CASE(EPI_QKV_ATTN)
        GEMM_CASE(EPI_SPLIT_GELU_ATTN)
        GEMM_CASE(EPI_SPLIT_SWIGLU_ATTN)
        default:
            return hipErrorInvalidValue;
    }
#undef GEMM_CASE
    return hipGetLastError();
}

// Rows [seq_len, l_pad) of q, k [heads, l_pad, D] and of v^T [heads, D,
// l_pad] (at their quad-swapped positions) as zeros: padded keys stay finite.
__global__ void zero_attn_pad_kernel(uint16_t* q, uint16_t* k, uint16_t* vt, int heads, int D, int seq_len,
                                     int l_pad) {
    const int pad = l_pad - seq_len;
    const size_t per = (size_t)heads * pad * D;   // elements per tensor
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < per; i += (size_t)gridDim.x * blockDim.x) {
        const int d = (int)(i % D);
        const size_t r = i / D;
        const int h = (int)(r / pad), t = seq_len + (int)(r % pad);
        q[((size_t)h * l_pad + t) * D + d] = 0;
        k[((size_t)h * l_pad + t) * D + d] = 0;
        const int qd = (t >> 2) & 3;
        const int pos = (t & ~15) | ((((qd & 1) << 1) | (qd >> 1)) << 2) | (t & 3);
        vt[((size_t)h * D + d) * l_pad + pos] = 0;
    }
}

hipError_t launch_zero_attn_pad(uint16_t* q, uint16_t* k, uint16_t* vt, int heads, int head_dim, int seq_len,
                                int l_pad, hipStream_t s) {
    if (l_pad <= seq_len) return hipSuccess;
    const size_t per = (size_t)heads * (l_pad - seq_len) * head_dim;
    const int blocks = (int)((per + 255) / 256 < 1024 ? (per + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_attn_pad_kernel, dim3(blocks), dim3(256), 0, s, q, k, vt, heads, head_dim, seq_len, l_pad);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    switch (a.wtype) {
        case MMDIT_BF16: return launch_gemm_t<MMDIT_BF16>(a, s);
        case MMDIT_INT8: return launch_gemm_t<MMDIT_INT8>(a, s);
        case MMDIT_F16: return launch_gemm_t<MMDIT_F16>(a, s);
        case MMDIT_FP8: return launch_gemm_t<MMDIT_FP8>(a, s);
        case WT_FP8_W16A: return launch_gemm_t<WT_FP8_W16A>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mmdit
