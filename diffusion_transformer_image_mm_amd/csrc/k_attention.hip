// Flash attention forward (no mask): O = softmax(Q K^T / sqrt(D)) V per head.
//
// Luminal blog, "The AMD MI300X pipeline" and "What the compiler found on its
// own": the attention sites of the diffusion transformer run as one fused
// kernel that computes softmax(QK^T)V tile by tile; the scaled-dot-product
// pattern is two matrix products, a scale, a max, an exponent, a sum and a
// divide. The transformer's attention has no mask.
//
// gfx950 design:
// * workgroup = 8 wavefronts x 32 query rows (256 rows of one head), two
//   wavefronts per SIMD (one wavefront per SIMD sustains only about half the
//   LDS read rate these tiles need); key/value tiles of 64 keys, each staged
//   in LDS once for all 256 rows: with 128-row workgroups (two per CU) every
//   tile was staged twice per CU, and the LDS pipe, which carries the tile
//   stores and ~125 B/clk of fragment reads, was the limit (FLUX double
//   block 1.408 -> 1.379 ms, single block 1.309 -> 1.279 ms, alternating
//   processes);
// * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as the first
//   operand, Q^T from registers as the second), so each lane holds 32 scores
//   of ONE query row: the row max needs one exchange between the wavefront's
//   halves (lane ^ 32, a register swap, no LDS round trip) and the row sum
//   none until the end;
// * online softmax in fp32 with exp2: scores are scaled by log2(e)/sqrt(D)
//   in one multiply-subtract against the row's current reference; the row
//   maximum is only taken (and the reference moved, when it grew by more than
//   2^8) on tiles where a lane's sum reaches 2^60 or is not finite: bf16
//   probabilities keep their precision at any magnitude, and most tiles skip
//   the maximum's ~25 VALU operations (attention alone 287 -> 279-285 us);
//   O is rescaled only by the lane's own factor, and only when the reference
//   moves;
// * O^T += V^T P^T: the probabilities are already in the second operand's
//   register layout (the key order inside one MFMA is free as long as both
//   operands agree); V^T is stored with the middle quads of every 16 keys
//   swapped, so a lane's 8 keys are one 16-byte LDS read (the 16 lanes served
//   together hit 16 distinct bank groups);
// * K and V^T tiles go global -> LDS with 16-byte direct-to-LDS loads into
//   two distinct LDS buffers (double buffering); chunk positions are
//   XOR-swizzled by row to spread LDS banks. The loads are written as
//   instructions (a wave-uniform base plus 32-bit lane offsets, the LDS
//   destination in m0): the compiler then counts the fragment reads exactly
//   and each MFMA waits only for its own operand, with the 16 fragment reads
//   of a phase issued four ahead of the MFMAs that consume them (with the
//   compiler's load builtin every MFMA waited for all reads in flight), and
//   the first four V^T fragments read before the softmax;
//   the kernel orders its LDS accesses itself with waits and barriers;
// * the last key tile masks keys >= seq_len to -inf; query rows >= seq_len
//   are computed on zero padding and not stored;
// * O is stored as fp16: it is the activation operand of the output
//   projection (values lie in the convex hull of V).
#include "common.h"

namespace mmdit {

namespace {
typedef __attribute__((address_space(3))) void lds_void;
MMDIT_DEV void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// 16-byte direct global -> LDS load (lane i writes lds_base + 16 i), written
// as an instruction so that the compiler's wait counting does not treat it as
// an LDS access of unknown extent.
MMDIT_DEV void g2l_16(const void* gsrc, lds_void* lds_base) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(gsrc) : "memory", "m0");
}
// PV phase with its first four V^T fragments already read (before the
// softmax): two reads, the four MFMAs on those, then read and MFMA
// alternately, then the last two MFMAs.
MMDIT_DEV void pv_schedule() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}
// Schedule of one 16-read, 16-MFMA phase: four reads ahead, then one MFMA and
// one read alternately, then the last four MFMAs.
MMDIT_DEV void read_ahead_schedule() {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // LDS reads
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}
}  // namespace

template <int D>
struct AttnTile {
    static constexpr int KV = 64;           // keys per tile
    static constexpr int RB = D * 2;        // bytes per K row
    static constexpr int CPR = D / 8;       // 16-byte chunks per K row
    static constexpr int K_RPI = 64 / CPR;  // K rows per wavefront load
    static constexpr int K_LPW = (KV / K_RPI) / 8;  // K loads per wavefront
    static constexpr int V_LPW = (D / 8) / 8;       // V^T loads per wavefront (8 rows each)
    static constexpr int K_BYTES = KV * RB;
    static constexpr int V_BYTES = D * KV * 2;
};

// One 64-key tile of the online softmax for the lane's query row (lane (r32, g)
// of a wavefront owning 32 query rows): S^T = K Q^T, the lazily rescaled
// exponentials, O^T += V^T P^T. K and V^T of tile t are in LDS (sK, sV).
template <int D>
MMDIT_DEV void attn_tile(int t, int seq_len, int g, const char* sK, const char* sV, const int (&k_off)[2][D / 16],
                         const int (&v_off)[D / 32][4], const bf16x8_t (&qf)[D / 16], f32x16_t (&o)[D / 32],
                         float& m_run, float& l_run, float c_log2) {
    using T = AttnTile<D>;
    // S^T = K Q^T for the two 32-key halves of the tile
    f32x16_t s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(sK + k_off[st][ds]);
            s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[st], 0, 0, 0);
        }
    }
    if constexpr (D == 128) read_ahead_schedule();
    // the first V^T fragments, read now so that the PV phase does not
    // start on an LDS round trip after the softmax
    bf16x8_t vpre[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) vpre[u] = *reinterpret_cast<const bf16x8_t*>(sV + v_off[0][u]);
    // element i of s[st]: key t*64 + st*32 + 8*(i/4) + 4g + i%4
    const int kv0 = t * T::KV;
    if (kv0 + T::KV > seq_len) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kv0 + st * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (key >= seq_len) s[st][i] = -INFINITY;
            }
    }
    // Exponentials against the current reference first. bf16 and fp32 share
    // their exponent range, so probabilities up to 2^60 above the reference
    // lose nothing; the row maximum (and a move of the reference) is only
    // needed when a lane's sum reaches 2^60 or is not finite (the first
    // tile, whose reference is -inf, or logits that jumped by ~60 in log2
    // units). O / l does not depend on which reference is used.
    float p[2][16];
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[st][i] = __builtin_amdgcn_exp2f(s[st][i] * c_log2 - m_run);
            psum += p[st][i];
        }
    float alpha = 1.0f;
    bool any_move = false;
    if (__ballot(!(psum < 0x1p60f)) != 0ull) {   // wave-uniform
        float tmax = s[0][0];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[st][i]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false,
                                                             false);
            tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float cand = tmax * c_log2;
        const bool move = cand > m_run + 8.0f;
        const float m_new = move ? cand : m_run;
        any_move = __ballot(move) != 0ull;
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        psum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[st][i] = __builtin_amdgcn_exp2f(s[st][i] * c_log2 - m_new);
                psum += p[st][i];
            }
    }
    bf16x8_t pf[4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) pf[st * 2 + (i >> 3)][i & 7] = static_cast<__bf16>(p[st][i]);
    l_run = l_run * alpha + psum;
    if (any_move) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bf16x8_t vf = dt == 0 ? vpre[u] : *reinterpret_cast<const bf16x8_t*>(sV + v_off[dt][u]);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[u], o[dt], 0, 0, 0);
        }
    if constexpr (D == 128) pv_schedule();
}

template <int D>
__global__ __launch_bounds__(512, 1) void attention_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ vt,
                                                           int seq_len, int l_pad, int heads,
                                                           uint16_t* __restrict__ out, int ldo,
                                                           float c_log2) {
    using T = AttnTile<D>;
    __shared__ __attribute__((aligned(1024))) char sK0[T::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char sV0[T::V_BYTES];
    __shared__ __attribute__((aligned(1024))) char sK1[T::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char sV1[T::V_BYTES];

    // Workgroups are dispatched round-robin over the 8 XCDs. Give each XCD a
    // contiguous range of (head, query-tile) pairs, so that the keys and
    // values of a head are read through one XCD's L2 (2.4 MB per head at
    // 4608 tokens) instead of all eight.
    const int nq = (seq_len + 255) / 256;
    const int total = nq * heads;
    int bid = blockIdx.x;
    if (total % 8 == 0) bid = (bid % 8) * (total / 8) + bid / 8;
    const int h = bid / nq, qt = bid % nq;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, r32 = lane & 31;
    const int qrow = qt * 256 + wave * 32 + r32;

    // ---- Q^T fragments (second MFMA operand): lane holds Q[qrow][ds*16 + 8g .. +7]
    const int qld = qrow < l_pad ? qrow : l_pad - 1;
    const uint16_t* qp = q + ((size_t)h * l_pad + qld) * D + g * 8;
    bf16x8_t qf[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) qf[ds] = *reinterpret_cast<const bf16x8_t*>(qp + ds * 16);
    // Q has landed before the loop: the compiler does not see the K/V loads,
    // so a first-use wait for Q inside the loop would wait for those instead.
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) asm volatile("" ::"v"(qf[ds]));

    // ---- load descriptors: wave-uniform head bases, 32-bit lane offsets
    // (l_pad < 2^24 keeps every offset below 2^32)
    const char* kbase = reinterpret_cast<const char*>(k + (size_t)h * l_pad * D);
    const char* vbase = reinterpret_cast<const char*>(vt + (size_t)h * D * l_pad);
    uint32_t k_src[T::K_LPW];
    int k_dst[T::K_LPW];
#pragma unroll
    for (int j = 0; j < T::K_LPW; ++j) {
        const int first = (wave * T::K_LPW + j) * T::K_RPI;
        const int r = first + lane / T::CPR;
        const int c = (lane % T::CPR) ^ (r & (T::CPR - 1));
        k_src[j] = (uint32_t)(r * D + c * 8) * 2u;
        k_dst[j] = first * T::RB;
    }
    uint32_t v_src[T::V_LPW];
    int v_dst[T::V_LPW];
#pragma unroll
    for (int j = 0; j < T::V_LPW; ++j) {
        const int first = (wave * T::V_LPW + j) * 8;
        const int d = first + lane / 8;
        const int c = (lane % 8) ^ ((d >> 1) & 7);
        v_src[j] = ((uint32_t)d * (uint32_t)l_pad + (uint32_t)(c * 8)) * 2u;
        v_dst[j] = first * 128;
    }
    auto issue = [&](int t, char* sK, char* sV) {
        const uint32_t koff = (uint32_t)t * T::KV * T::RB;  // bytes along the key rows
        const uint32_t voff = (uint32_t)t * T::KV * 2;      // bytes along a V^T row
#pragma unroll
        for (int j = 0; j < T::K_LPW; ++j) g2l_16(kbase + (k_src[j] + koff), (lds_void*)(sK + k_dst[j]));
#pragma unroll
        for (int j = 0; j < T::V_LPW; ++j) g2l_16(vbase + (v_src[j] + voff), (lds_void*)(sV + v_dst[j]));
    };

    // ---- fragment offsets
    int k_off[2][D / 16];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const int row = st * 32 + r32;
            const int c = ds * 2 + g;
            k_off[st][ds] = row * T::RB + ((c ^ (row & (T::CPR - 1))) * 16);
        }
    // V^T fragment u of lane (r32, g): keys 16u + 4g + {0..3, 8..11}, which the
    // quad-swapped layout stores as chunk 2u + g of row d
    int v_off[D / 32][4];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int d = dt * 32 + r32;
            const int c = 2 * u + g;
            v_off[dt][u] = d * 128 + ((c ^ ((d >> 1) & 7)) * 16);
        }

    f32x16_t o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int nkv = (seq_len + T::KV - 1) / T::KV;

    auto compute = [&](int t, const char* sK, const char* sV) {
        attn_tile<D>(t, seq_len, g, sK, sV, k_off, v_off, qf, o, m_run, l_run, c_log2);
    };

    issue(0, sK0, sV0);
    wait_vmcnt0();
    __syncthreads();
    for (int t = 0; t < nkv; t += 2) {
        if (t + 1 < nkv) issue(t + 1, sK1, sV1);
        compute(t, sK0, sV0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt0();
        __syncthreads();
        if (t + 1 >= nkv) break;
        if (t + 2 < nkv) issue(t + 2, sK0, sV0);
        compute(t + 1, sK1, sV1);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt0();
        __syncthreads();
    }

    // ---- normalise and store: o[dt] element i is O[qrow][dt*32 + 8*(i/4) + 4g + i%4]
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (qrow < seq_len) {
        uint16_t* op = out + (size_t)qrow * ldo + h * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const uint2 w = make_uint2(pack2h(o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv),
                                           pack2h(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv));
                *reinterpret_cast<uint2*>(op + dt * 32 + 8 * i4) = w;
            }
    }
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int heads,
                            int seq_len, int head_dim, int l_pad, uint16_t* out, int ldo,
                            hipStream_t s) {
    if (seq_len <= 0) return hipSuccess;
    if (l_pad >= (1 << 24)) return hipErrorInvalidValue;   // 32-bit load offsets
    dim3 grid(((seq_len + 255) / 256) * heads), block(512);
    const float c_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
    if (head_dim == 128)
        hipLaunchKernelGGL(attention_kernel<128>, grid, block, 0, s, q, k, vt, seq_len, l_pad, heads, out, ldo,
                           c_log2);
    else if (head_dim == 64)
        hipLaunchKernelGGL(attention_kernel<64>, grid, block, 0, s, q, k, vt, seq_len, l_pad, heads, out, ldo,
                           c_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mmdit
