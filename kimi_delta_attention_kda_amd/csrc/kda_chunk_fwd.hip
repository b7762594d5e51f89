// kda_chunk_fwd.hip -- chunkwise KDA prefill for gfx950 (CDNA4).
//
// Pages cited by title and section:
//   [TL-KDA]  "TileLang 实战：KDA 从零到一 -- Chunked 线性注意力": section 1
//             (recurrence, (d_v, d_k) state), section 6.4 (sequence axis kept
//             out of the grid: the state is carried through a sequential chunk
//             loop), 6.4.1 (split d_v, never d_k), 6.4.2 (state update after
//             the chunk's output write-back), 6.4.3 (log-domain gate).
//   [FKDA-LM] "FlashKDA 里的 L 矩阵和 Mqk 矩阵是什么": paragraphs "30秒速览"
//             (U, out and state-advance formulas), "L 矩阵的构造" (strictly
//             lower, row-scaled by beta), "Mqk 矩阵的构造" (lower including the
//             diagonal), "为什么 CHUNK16" (L^16 = 0, inverse by Neumann
//             squaring with 6 16x16 products), "K2 内核如何消费" (the four
//             steps and the state advance reusing U; prep and recurrence as
//             two roles that exchange per-chunk operands).
//   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)": gate and beta formulas.
//
// Per chunk of C = 16 tokens of one (sequence, head), with G the chunk-local
// cumulative gate (G_i = sum_{j<=i} g_j, per channel) and S the state as
// (d_k x d_v) = S^T of the (d_v, d_k) layout:
//   k~ = k e^G, q~ = q e^G, k^r = k e^{G_C - G}
//   L_ij   = -beta_i sum_c k_ic k_jc e^{G_ic - G_jc}   (i > j)
//   Mqk_ij =         sum_c q_ic k_jc e^{G_ic - G_jc}   (i >= j)
//   INV = (I - L)^{-1} = (I + L)(I + L^2)(I + L^4)(I + L^8)
//   u = beta (v - k~ S);  U = INV u;  O = scale (q~ S + Mqk U)
//   S <- Diag(e^{G_C}) S + k^r^T U     (after the output)
// Sign of L: the recurrence gives (I + A) U = u with A_ij = beta_i <k~_i, k_j e^{-G_j}>,
// so L := -A and U = (I - L)^{-1} u (the page prints the series both ways).
//
// Work split on MI355X.  Everything that does not depend on the state (the
// gate, the decayed operands, L, Mqk, INV: the "prep") is produced by
// PRODUCER workgroups; the state recurrence runs in CONSUMER workgroups, one
// per d_v slab of BDV columns, each holding its fp32 state slab in MFMA
// accumulators for the whole walk over the sequence.  One TEAM = NS consumer
// workgroups + NP producer workgroups for one (sequence, head) chain at a
// time.  Each producer wave builds whole chunks on its own and writes a
// ~15 KiB payload, already in MFMA fragment order, into a ring of RING slots
// in device memory; every consumer workgroup of the team copies each payload
// into LDS (one chunk ahead) and consumes it.  The prep therefore runs once
// per chunk for all d_v slabs, spread over the team's producer waves, instead
// of once per slab.
//
// Ring protocol.  All workgroups of a team share blockIdx % 8, i.e. run on the
// same XCD and share its L2 (MI355X dispatches workgroups to its 8 XCDs round
// robin).  A producer writes the payload with ordinary stores, waits for them
// (s_waitcnt vmcnt(0): stores are acknowledged by L2), then stores the slot's
// ready flag with an L2-coherent (sc1) store.  A consumer polls the flag with
// L2-coherent loads, invalidates its L1 (buffer_inv sc0, which only touches
// the CU-local cache) and copies the payload.  After the copy it adds 1 to
// the slot's use counter; a producer reuses a slot once all NS consumers have
// copied it.  No device-scope cache write-back or L2 invalidation is needed.
// Every wait is bounded; on timeout the kernel sets an error word and stops
// waiting, so it always terminates.  All workgroups of the grid must be
// resident at once; the host sizes the grid from the occupancy query.
//
// Overflow-safe L / Mqk.  The factored form <k_i e^{G_i}, k_j e^{-G_j}> leaves
// the fp32 range once a channel decays by more than ~88 nats inside a chunk.
// A chunk in which every channel's total decay is at most 100 in log2 units
// ("mild") uses one reference at the chunk end:
//   rows k_i 2^{g_C - g_i} (<= 2^100), columns k^r_j = k_j 2^{g_j - g_C} (<= 1).
// Other chunks use four 4-token blocks: for rows in block b the reference is
// the cumulative decay g' at the end of block b-1, with each token's decay
// clipped at 24 (e^g floored at 2^-24):
//   rows k_i 2^{g'_ref - g'_i} (<= 1),  columns k_j 2^{g'_j - g'_ref} (<= 2^72
//   inside block b, <= 1 before it),
// one MFMA pass per row block.  Pairs whose true decay gap exceeds 24 (log2)
// are then computed as at most 2^-24 instead of their (smaller) true value,
// an error below fp32 rounding of the O(1) entries; everything else is exact.
// The state-side operands (k~, q~, k^r) and the state decay use the unclipped
// gates; all their factors are <= 1, so underflow only drops negligible terms.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int CH = 16;              // chunk length (tokens)
constexpr int NTHR = 256;           // threads per workgroup (4 waves), both roles
constexpr int NPW = 4;              // producer waves per producer workgroup
constexpr long SPIN_LIMIT = 1L << 20;   // polls (each an L2 round trip plus a short sleep): ~1 s

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ ring sync
__device__ __forceinline__ int ld_flag(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_flag(int *p, int v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait (wave-uniform) until *p >= v; false on timeout or an earlier timeout.
__device__ bool wait_geq(const int *p, int v, int *err) {
    if (ld_flag(err)) return false;
    for (long n = 0; ld_flag(p) < v; ++n) {
        __builtin_amdgcn_s_sleep(2);
        if (n > SPIN_LIMIT) { st_flag(err, 1); return false; }
    }
    return true;
}
__device__ __forceinline__ void stores_done() {   // all of this wave's stores reached L2
    __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
    asm volatile("" ::: "memory");
}
// 16 bytes per lane from global memory straight into LDS (gfx950 LDS DMA): lane i
// writes LDS bytes [lds + 16 i, lds + 16 i + 16).  `lds` must be wave-uniform.
// The load is agent-coherent (sc1), so it reads L2 and never a stale L1 line.
// Completion is counted by vmcnt; M0 is restored afterwards.
__device__ __forceinline__ void lds_dma16(const void *src, unsigned lds) {
    unsigned saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off sc1\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {       // at most N vector-memory ops of this wave in flight
    static_assert(N >= 0 && N < 16, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void sched_fence() {   // no instruction moves across this point
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void lds_done() {      // this wave's LDS ops completed
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0)
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------ payload layout
// Fragment coordinates: lane = 16 lq + ln.  16x16 MFMA layouts:
//   A (16 x K): lane holds row ln, K slice lq;  B (K x 16): column ln, K slice lq;
//   C (16 x 16): rows 4lq .. 4lq+3 of column ln.
// bf16: KD/QD fragment s (32 channels): lane 16 B = channels {32s+4lq+i, 32s+16+4lq+i};
//       KR fragment mt: lane 8 B = k^r[16mt+ln][4lq .. 4lq+3];
//       INV/MQK: lane 16 B = {hi(X[ln][4lq+i]), lo(X[ln][4lq+i])}.
// f32:  KD/QD fragment mt: lane 16 B = channels 16mt+4lq+i;  KR fragment mt:
//       lane 16 B = k^r[16mt+ln][4lq+i];  INV/MQK: lane 16 B = X[ln][4lq+i].
// Both: BETA[16] and EG[dk] fp32; V fragment vt: lane = v[4lq .. 4lq+3][16vt+ln]
//       in the activation dtype (the consumer's C layout).
template <bool BF16, int DK, int DV>
struct PL {
    static constexpr int MT = DK / 16;
    static constexpr int NF = BF16 ? DK / 32 : DK / 16;   // KD/QD fragments
    static constexpr int KRB = BF16 ? 8 : 16;             // bytes per lane per KR fragment
    static constexpr int ES = BF16 ? 2 : 4;               // activation element size
    static constexpr int KD = 0;
    static constexpr int QD = KD + NF * 64 * 16;
    static constexpr int KR = QD + NF * 64 * 16;
    static constexpr int INV = KR + MT * 64 * KRB;
    static constexpr int MQK = INV + 64 * 16;
    static constexpr int BETA = MQK + 64 * 16;
    static constexpr int EG = BETA + 64;
    static constexpr int V = EG + DK * 4;                  // v: fragment vt, lane: rows 4lq..4lq+3 of column 16vt+ln
    static constexpr int END = V + (DV / 16) * 64 * 4 * ES;
    static constexpr int BYTES = (END + 1023) / 1024 * 1024;   // copied size
};
static_assert(PL<true, 128, 128>::BYTES <= KDA_RING_SLOT_BYTES, "payload too large");
static_assert(PL<false, 64, 128>::BYTES <= KDA_RING_SLOT_BYTES, "payload too large");

template <bool BF16> struct Elem;
template <> struct Elem<true> { using T = uint16_t; };
template <> struct Elem<false> { using T = float; };

template <bool BF16>
__device__ __forceinline__ float load_act(const void *p, size_t i) {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void store_act(void *p, size_t i, float x) {
    if constexpr (BF16) static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    else static_cast<float *>(p)[i] = x;
}
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::T to_elem(float x) {
    if constexpr (BF16) return f32_to_bf16(x);
    else return x;
}

// bf16 hi/lo split of 4 values into one 8-wide operand [hi0..hi3, lo0..lo3].
__device__ __forceinline__ bf16x8 split_hilo(f32x4 x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 hi = static_cast<__bf16>(x[i]);
        r[i] = hi;
        r[4 + i] = static_cast<__bf16>(x[i] - static_cast<float>(hi));
    }
    return r;
}
// A operand pairing with split_hilo B operands: the row values (hi or lo part)
// repeated in both K halves.
__device__ __forceinline__ bf16x8 dup4(bf16x4 a) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = a[i]; }
    return r;
}
__device__ __forceinline__ void hilo4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = static_cast<__bf16>(x[i]);
        lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hi[i]));
    }
}

// --------------------------------------------------------------- team layout
struct Role {
    int team;      // team id, or -1 when idle
    int member;    // 0 .. NS-1 consumer (slab), NS .. NS+NP-1 producer
};
__device__ __forceinline__ Role role_of(int NS, int NP, int n_teams) {
    const int TS = NS + NP;
    const int x = blockIdx.x % 8, y = blockIdx.x / 8;
    Role r;
    r.team = (y / TS) * 8 + x;
    r.member = y % TS;
    if (r.team >= n_teams) r.team = -1;
    return r;
}

struct ChainInfo {
    size_t bos;
    int len, seq, head;
};
__device__ __forceinline__ ChainInfo chain_info(const ChunkArgs &a, int chain) {
    ChainInfo c;
    c.seq = chain / a.H;
    c.head = chain - c.seq * a.H;
    if (a.cu_seqlens) {
        c.bos = (size_t)a.cu_seqlens[c.seq];
        c.len = a.cu_seqlens[c.seq + 1] - a.cu_seqlens[c.seq];
    } else {
        c.bos = (size_t)c.seq * a.T;
        c.len = a.T;
    }
    return c;
}

// ============================================================== producer
// A producer CREW of DK/64 waves (2 for d_k = 128) builds one chunk: each wave
// owns 64 channels (one per lane) for all 16 tokens, writes its part of the
// payload, and contracts its channels' share of L and Mqk.  The second wave
// hands its partial 16x16 sums to the first (the "lead") through LDS; the lead
// adds them, applies the masks and beta, forms INV and writes the rest.
constexpr int CW = 64;   // channels per producer wave

template <bool BF16>
struct ProdScratch {   // per producer wave, in LDS
    using E = typename Elem<BF16>::T;
    static constexpr int PK = CW + (BF16 ? 8 : 4);
    alignas(16) E R[CH][PK];     // k rows of the L / Mqk contraction
    alignas(16) E Rq[CH][PK];    // q rows
    alignas(16) E Cv[CH][PK];    // columns of the current pass
    alignas(16) float X[CH][CH + 1];
    alignas(16) float Pm[CH][CH + 1];
    alignas(16) float beta[CH];
    alignas(16) f32x4 partL[64];  // partial sums handed to the lead wave
    alignas(16) f32x4 partM[64];
    int flag;                     // sequence number of the posted partials
    int ack;                      // sequence number the lead has consumed
};

// One chunk's inputs for one producer wave: channel `lane` of its half
// (k, q, g_raw) and its value columns, 16 tokens, kept as loaded.
template <bool BF16, int DV, int NVW>
struct ProdIn {
    using Raw = typename std::conditional<BF16, uint32_t, float>::type;
    Raw k[CH], q[CH], a[CH];
    Raw v[CH][NVW];
    float b;   // beta_raw of token `lane` for lanes < 16 (lead wave)
    __device__ __forceinline__ static float get(Raw r) {
        if constexpr (BF16) return bf16_to_f32((uint16_t)r);
        else return r;
    }
};

template <bool BF16>
__device__ __forceinline__ typename std::conditional<BF16, uint32_t, float>::type
ld_one(const void *p, size_t off) {
    if constexpr (BF16) return static_cast<const uint16_t *>(p)[off];
    else return static_cast<const float *>(p)[off];
}

// Loads of one chunk: part 0 = k, g_raw (needed first), part 1 = q, v, beta_raw.
template <int PART, bool BF16, int DK, int DV, int NVW>
__device__ __forceinline__ void prod_load(ProdIn<BF16, DV, NVW> &in, const ChunkArgs &a, size_t tok0,
                                          int rem, int h, int c, int vbase, int nvcol, int lane, bool lead) {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        const size_t row = (tok0 + t) * a.H + h;
        const bool live = t < rem;
        if constexpr (PART == 0) {
            in.k[t] = live ? ld_one<BF16>(a.k, row * DK + c) : 0;
            in.a[t] = live ? ld_one<BF16>(a.g_raw, row * DK + c) : 0;
        } else {
            in.q[t] = live ? ld_one<BF16>(a.q, row * DK + c) : 0;
#pragma unroll
            for (int j = 0; j < NVW; ++j) {
                const int vc = lane + 64 * j;
                in.v[t][j] = (live && vc < nvcol) ? ld_one<BF16>(a.v, row * DV + vbase + vc) : 0;
            }
        }
    }
    if constexpr (PART == 1)
        in.b = (lead && lane < rem) ? load_act<BF16>(a.beta_raw, (tok0 + lane) * a.H + h) : 0.f;
}

// C (16x16, C layout) += A B with A rows from LDS matrix Am (row-major, stride
// CH+1) and B in C layout (registers); hi/lo bf16 splits on both sides
// (error ~2^-16 relative).
__device__ __forceinline__ f32x4 mm16_lds_reg(const float (*Am)[CH + 1], f32x4 B, f32x4 acc,
                                              int ln, int lq) {
    f32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = Am[ln][4 * lq + i];
    bf16x4 ahi, alo;
    hilo4(a, ahi, alo);
    const bf16x8 b = split_hilo(B);
    acc = mfma_bf16(dup4(ahi), b, acc);
    acc = mfma_bf16(dup4(alo), b, acc);
    return acc;
}
__device__ __forceinline__ void st_rows(float (*Dm)[CH + 1], f32x4 c, int ln, int lq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Dm[4 * lq + i][ln] = c[i];
}
// fp32 path: D += A B with both operands from LDS, 4 fp32 MFMAs.
__device__ __forceinline__ f32x4 mm16_f32(const float (*A)[CH + 1], const float (*B)[CH + 1],
                                          f32x4 acc, int ln, int lq) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_f32(A[ln][4 * s + lq], B[4 * s + lq][ln], acc);
    return acc;
}

// acc += rows(A) x cols(B)^T over the wave's 64 channels, both from LDS
// [token][channel]; columns with token index > cmax read as zero.
template <bool BF16, typename E, int PK>
__device__ __forceinline__ f32x4 contract64(const E (*A)[PK], const E (*B)[PK], int cmax,
                                            f32x4 acc, int ln, int lq) {
    const bool live = ln <= cmax;
    if constexpr (BF16) {
#pragma unroll
        for (int s = 0; s < CW / 32; ++s) {
            const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&A[ln][32 * s + 8 * lq]);
            bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&B[ln][32 * s + 8 * lq]);
            if (!live) bv = bf16x8{};
            acc = mfma_bf16(av, bv, acc);
        }
    } else {
#pragma unroll
        for (int s = 0; s < CW / 4; ++s) {
            const float bv = live ? B[ln][4 * s + lq] : 0.f;
            acc = mfma_f32(A[ln][4 * s + lq], bv, acc);
        }
    }
    return acc;
}

__device__ __forceinline__ bool lds_wait_geq(const int *p, int v, int *err) {
    for (long n = 0; *reinterpret_cast<const volatile int *>(p) < v; ++n) {
        __builtin_amdgcn_s_sleep(1);
        if (n > SPIN_LIMIT) { st_flag(err, 1); return false; }
    }
    asm volatile("" ::: "memory");
    return true;
}

// Produce this wave's half of one chunk's payload into ring slot `slot`.
// `c` = this lane's channel; `hf` = half (0 = lead); `seq` = chunk number + 1.
template <bool BF16, int DK, int DV, int NVW>
__device__ void produce_half(const ProdIn<BF16, DV, NVW> &in, int rem, float A_exp, float dtl,
                             ProdScratch<BF16> &me, ProdScratch<BF16> &mate, unsigned char *slot,
                             int lane, int hf, int vbase, int nvcol, int seq, int &posted, int *err) {
    constexpr int NPAIR = DK / 64;
    using P = PL<BF16, DK, DV>;
    using In = ProdIn<BF16, DV, NVW>;
    const int ln = lane & 15, lq = lane >> 4;
    const int c = CW * hf + lane;

    // ---- v, re-laid out as the consumers' C-layout fragments
#pragma unroll
    for (int j = 0; j < NVW; ++j) {
        const int vc = vbase + lane + 64 * j;
        if (lane + 64 * j < nvcol) {
            const int vt = vc >> 4, vl = vc & 15;
#pragma unroll
            for (int fq = 0; fq < 4; ++fq) {
                if constexpr (BF16) {
                    uint2 w;
                    w.x = (in.v[4 * fq][j] & 0xffffu) | (in.v[4 * fq + 1][j] << 16);
                    w.y = (in.v[4 * fq + 2][j] & 0xffffu) | (in.v[4 * fq + 3][j] << 16);
                    *reinterpret_cast<uint2 *>(slot + P::V + ((vt * 64 + fq * 16 + vl) * 4) * 2) = w;
                } else {
                    const f32x4 w = {in.v[4 * fq][j], in.v[4 * fq + 1][j], in.v[4 * fq + 2][j], in.v[4 * fq + 3][j]};
                    *reinterpret_cast<f32x4 *>(slot + P::V + ((vt * 64 + fq * 16 + vl) * 4) * 4) = w;
                }
            }
        }
    }

    // ---- gate: e^{g} = 2^{-A log2(1 + 2^{x log2e})}; padded tokens do not decay
    float al[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        const float y = __builtin_fmaf(In::get(in.a[t]), kLog2e, dtl);
        const float sp2 = y > 20.0f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
        al[t] = t < rem ? __builtin_amdgcn_exp2f(-A_exp * sp2) : 1.f;
    }
    if (hf == 0 && lane < CH) me.beta[lane] = lane < rem ? sigmoid_f(in.b) : 0.f;

    // ---- k~, q~ (prefix products), e^{G_C}, k^r (suffix products)
    float p = 1.f;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        p *= al[t];
        const float kd = In::get(in.k[t]) * p, qd = In::get(in.q[t]) * p;
        if constexpr (BF16) {
            const int off = (((c >> 5) * 4 + ((c >> 2) & 3)) * 16 + t) * 16 + (4 * ((c >> 4) & 1) + (c & 3)) * 2;
            *reinterpret_cast<uint16_t *>(slot + P::KD + off) = f32_to_bf16(kd);
            *reinterpret_cast<uint16_t *>(slot + P::QD + off) = f32_to_bf16(qd);
        } else {
            const int off = (((c >> 4) * 4 + ((c >> 2) & 3)) * 16 + t) * 16 + (c & 3) * 4;
            *reinterpret_cast<float *>(slot + P::KD + off) = kd;
            *reinterpret_cast<float *>(slot + P::QD + off) = qd;
        }
    }
    const float Pc = p;
    reinterpret_cast<float *>(slot + P::EG)[c] = Pc;
    float kr[CH];
    {
        float sq = 1.f;
#pragma unroll
        for (int t = CH - 1; t >= 0; --t) {
            kr[t] = In::get(in.k[t]) * sq;
            sq *= al[t];
        }
    }
    {
        const int mt = c >> 4, cl = c & 15;
#pragma unroll
        for (int fq = 0; fq < 4; ++fq) {
            if constexpr (BF16) {
                uint2 v;
                v.x = pack_bf16x2(kr[4 * fq], kr[4 * fq + 1]);
                v.y = pack_bf16x2(kr[4 * fq + 2], kr[4 * fq + 3]);
                *reinterpret_cast<uint2 *>(slot + P::KR + ((mt * 4 + fq) * 16 + cl) * 8) = v;
            } else {
                const f32x4 v = {kr[4 * fq], kr[4 * fq + 1], kr[4 * fq + 2], kr[4 * fq + 3]};
                *reinterpret_cast<f32x4 *>(slot + P::KR + ((mt * 4 + fq) * 16 + cl) * 16) = v;
            }
        }
    }

    // ---- this wave's share of L and Mqk (each wave picks its own scheme)
    const bool mild = __all(Pc >= 0x1p-100f);
    f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
    if (mild) {
        // one reference at the chunk end: rows k 2^{g_C - g}, q 2^{g_C - g}; columns k^r
        float pr = __builtin_amdgcn_rcpf(Pc);
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            pr *= al[t];
            me.R[t][lane] = to_elem<BF16>(In::get(in.k[t]) * pr);
            me.Rq[t][lane] = to_elem<BF16>(In::get(in.q[t]) * pr);
            me.Cv[t][lane] = to_elem<BF16>(kr[t]);
        }
        lds_done();
        accL = contract64<BF16>(me.R, me.Cv, CH - 1, accL, ln, lq);
        accM = contract64<BF16>(me.Rq, me.Cv, CH - 1, accM, ln, lq);
    } else {
        // four token blocks, decay clipped at 2^-24 per token; rows relative to
        // the start of their own block
        float ac[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) ac[t] = fmaxf(al[t], 0x1p-24f);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float lp = 1.f;
#pragma unroll
            for (int t = 4 * b; t < 4 * b + 4; ++t) {
                lp *= ac[t];
                me.R[t][lane] = to_elem<BF16>(In::get(in.k[t]) * lp);
                me.Rq[t][lane] = to_elem<BF16>(In::get(in.q[t]) * lp);
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // columns for row block b: own block k 2^{g'_t - g'_ref}; earlier
            // tokens k 2^{g'_t - g'_ref} <= 1 (products of the clipped decays after t)
            float lp = 1.f;
#pragma unroll
            for (int t = 4 * b; t < 4 * b + 4; ++t) {
                lp *= ac[t];
                me.Cv[t][lane] = to_elem<BF16>(In::get(in.k[t]) * __builtin_amdgcn_rcpf(lp));
            }
            float F = 1.f;
#pragma unroll
            for (int t = 4 * b - 1; t >= 0; --t) {
                me.Cv[t][lane] = to_elem<BF16>(In::get(in.k[t]) * F);
                F *= ac[t];
            }
            lds_done();
            const f32x4 pl = contract64<BF16>(me.R, me.Cv, 4 * b + 3, f32x4{0.f, 0.f, 0.f, 0.f}, ln, lq);
            const f32x4 pm = contract64<BF16>(me.Rq, me.Cv, 4 * b + 3, f32x4{0.f, 0.f, 0.f, 0.f}, ln, lq);
            if (lq == b) { accL = pl; accM = pm; }
            lds_done();   // every lane has read Cv before the next variant overwrites it
        }
    }

    // ---- combine the crew's partial sums in the lead wave
    if constexpr (NPAIR == 2) {
        if (hf == 1) {
            stores_done();                       // this wave's payload is in L2
            lds_wait_geq(&me.ack, posted, err);  // lead consumed the previous partials
            me.partL[lane] = accL;
            me.partM[lane] = accM;
            lds_done();
            *reinterpret_cast<volatile int *>(&me.flag) = seq;
            posted = seq;
            return;
        }
        lds_wait_geq(&mate.flag, seq, err);
        lds_done();
        const f32x4 oL = mate.partL[lane], oM = mate.partM[lane];
        lds_done();
        *reinterpret_cast<volatile int *>(&mate.ack) = seq;
#pragma unroll
        for (int i = 0; i < 4; ++i) { accL[i] += oL[i]; accM[i] += oM[i]; }
    }
    lds_done();
    f32x4 L, M;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lq + i;
        L[i] = r > ln ? -me.beta[r] * accL[i] : 0.f;
        M[i] = r >= ln ? accM[i] : 0.f;
    }

    // ---- INV = (I + L)(I + L^2)(I + L^4)(I + L^8)
    f32x4 X;
#pragma unroll
    for (int i = 0; i < 4; ++i) X[i] = (4 * lq + i == ln ? 1.f : 0.f) + L[i];
    if constexpr (BF16) {
        f32x4 Pw = L;
        st_rows(me.Pm, Pw, ln, lq);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            lds_done();
            const f32x4 P2 = mm16_lds_reg(me.Pm, Pw, f32x4{0.f, 0.f, 0.f, 0.f}, ln, lq);
            st_rows(me.X, X, ln, lq);
            lds_done();
            X = mm16_lds_reg(me.X, P2, X, ln, lq);
            Pw = P2;
            st_rows(me.Pm, Pw, ln, lq);
        }
    } else {
        st_rows(me.Pm, L, ln, lq);
        st_rows(me.X, X, ln, lq);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            lds_done();
            const f32x4 P2 = mm16_f32(me.Pm, me.Pm, f32x4{0.f, 0.f, 0.f, 0.f}, ln, lq);
            lds_done();
            st_rows(me.Pm, P2, ln, lq);
            lds_done();
            X = mm16_f32(me.X, me.Pm, X, ln, lq);
            lds_done();
            st_rows(me.X, X, ln, lq);
        }
    }
    // ---- INV and Mqk as A fragments (row ln, columns 4lq .. 4lq+3)
    lds_done();
    st_rows(me.X, X, ln, lq);
    st_rows(me.Pm, M, ln, lq);
    lds_done();
    f32x4 xi, mi;
#pragma unroll
    for (int i = 0; i < 4; ++i) { xi[i] = me.X[ln][4 * lq + i]; mi[i] = me.Pm[ln][4 * lq + i]; }
    if constexpr (BF16) {
        bf16x4 h, l;
        hilo4(xi, h, l);
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = h[i]; v[4 + i] = l[i]; }
        *reinterpret_cast<bf16x8 *>(slot + P::INV + lane * 16) = v;
        hilo4(mi, h, l);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = h[i]; v[4 + i] = l[i]; }
        *reinterpret_cast<bf16x8 *>(slot + P::MQK + lane * 16) = v;
    } else {
        *reinterpret_cast<f32x4 *>(slot + P::INV + lane * 16) = xi;
        *reinterpret_cast<f32x4 *>(slot + P::MQK + lane * 16) = mi;
    }
    if (lane < CH) reinterpret_cast<float *>(slot + P::BETA)[lane] = me.beta[lane];
}

// ============================================================== the kernel
__device__ __forceinline__ void lds_barrier() {   // LDS-only barrier: global ops stay in flight
    lds_done();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <bool BF16, int DK, int DV, int BDV>
__global__ __launch_bounds__(NTHR, 2) void chunk_fwd_kernel(ChunkArgs args)
{
    using P = PL<BF16, DK, DV>;
    constexpr int NS = DV / BDV;
    constexpr int NCW = BDV / 16;          // compute waves of a consumer workgroup
    constexpr int MT = DK / 16;
    constexpr int NP = KDA_PRODUCER_WGS;
    constexpr int NPAIR = DK / CW;         // waves per producer crew
    constexpr int NVW = (DV / NPAIR + 63) / 64;   // value columns per producer lane
    static_assert(NCW >= 1 && NCW <= 4, "consumer slab of 16..64 columns");
    static_assert(KDA_RING <= 64, "one lane per ring slot when polling");

    // LDS: producers use 4 scratch areas, consumers a 3-deep payload buffer.
    constexpr int PROD_BYTES = (int)sizeof(ProdScratch<BF16>) * NPW;
    constexpr int CONS_BYTES = 3 * ((P::BYTES + 16 * NTHR - 1) / (16 * NTHR)) * 16 * NTHR;
    constexpr int LDS_BYTES = PROD_BYTES > CONS_BYTES ? PROD_BYTES : CONS_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    const Role role = role_of(NS, NP, args.n_teams);
    if (role.team < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;
    unsigned char *ring = args.ring + (size_t)role.team * KDA_RING * KDA_RING_SLOT_BYTES;
    int *ready = args.ready + role.team * KDA_RING;
    int *used = args.used + role.team * KDA_RING;
    int *err = args.err;
    const int n_chains = args.n_seq * args.H;

    if (role.member >= NS) {
        // ======================================================= producer
        auto *scr = reinterpret_cast<ProdScratch<BF16> *>(lds);
        if (lane == 0) { scr[w].flag = 0; scr[w].ack = 0; }
        __syncthreads();
        const int hf = w % NPAIR;                                  // half of the crew
        const int crew = (role.member - NS) * (NPW / NPAIR) + w / NPAIR;
        constexpr int STEP = NP * (NPW / NPAIR);                   // crews per team
        ProdScratch<BF16> &me = scr[w];
        ProdScratch<BF16> &mate = scr[w ^ (NPAIR - 1)];
        const int c = CW * hf + lane;
        const int nvcol = DV / NPAIR, vbase = nvcol * hf;
        int q_base = 0, posted = 0;
        ProdIn<BF16, DV, NVW> cur;
        for (int chain = role.team; chain < n_chains; chain += args.n_teams) {
            const ChainInfo ci = chain_info(args, chain);
            const int nch = (ci.len + CH - 1) / CH;
            const float A_exp = expf(args.A_log[ci.head]);
            const float dtl = args.dt_bias[(size_t)ci.head * DK + c] * kLog2e;
            int q = q_base + ((crew - q_base) % STEP + STEP) % STEP;
            if (q < q_base + nch) {
                const int cc = q - q_base;
                prod_load<0, BF16, DK, DV, NVW>(cur, args, ci.bos + (size_t)cc * CH, min(CH, ci.len - cc * CH),
                                                ci.head, c, vbase, nvcol, lane, hf == 0);
            }
            for (; q < q_base + nch; q += STEP) {
                const int cc = q - q_base;
                const int rem = min(CH, ci.len - cc * CH);
                // this chunk's q, v, beta_raw, then the next chunk's k, g_raw:
                // both overlap the slot wait and this chunk's gate
                prod_load<1, BF16, DK, DV, NVW>(cur, args, ci.bos + (size_t)cc * CH, rem, ci.head, c, vbase,
                                                nvcol, lane, hf == 0);
                ProdIn<BF16, DV, NVW> nxt;
                const int cn = cc + STEP;
                if (cn < nch)
                    prod_load<0, BF16, DK, DV, NVW>(nxt, args, ci.bos + (size_t)cn * CH, min(CH, ci.len - cn * CH),
                                                    ci.head, c, vbase, nvcol, lane, hf == 0);
                const int s = q % KDA_RING;
                if (q >= KDA_RING) wait_geq(&used[s], NS * (q / KDA_RING), err);
                produce_half<BF16, DK, DV, NVW>(cur, rem, A_exp, dtl, me, mate,
                                                ring + (size_t)s * KDA_RING_SLOT_BYTES, lane, hf, vbase, nvcol,
                                                q + 1, posted, err);
                if (hf == 0) {
                    stores_done();   // lead's stores; the other half drained before posting
                    if (lane == 0) st_flag(&ready[s], q + 1);
                }
#pragma unroll
                for (int t = 0; t < CH; ++t) { cur.k[t] = nxt.k[t]; cur.a[t] = nxt.a[t]; }
            }
            q_base += nch;
        }
        return;
    }

    // =========================================================== consumer
    const int slab = role.member;
    const bool computes = w < NCW;
    const int v0 = slab * BDV + 16 * (w < NCW ? w : 0);
    const int vt = v0 >> 4;
    int q_total = 0;
    for (int chain = role.team; chain < n_chains; chain += args.n_teams)
        q_total += (chain_info(args, chain).len + CH - 1) / CH;

    // Ready tracking: chunks <= known are ready.  One poll loads all RING flags
    // (one lane per slot) and extends `known` over the run of ready chunks.
    int known = -1;
    auto ensure_ready = [&](int need) {
        if (need <= known) return;
        if (ld_flag(err)) return;
        for (long n = 0;; ++n) {
            const int f = lane < KDA_RING ? ld_flag(&ready[lane]) : 0;
            const int cj = need + lane;
            const int fj = __shfl(f, cj % KDA_RING);
            const unsigned long long ok = __ballot(lane < KDA_RING && fj >= cj + 1);
            const int run = __builtin_ctzll(~ok);
            if (run > 0) { known = need + run - 1; return; }
            __builtin_amdgcn_s_sleep(2);
            if (n > SPIN_LIMIT) { st_flag(err, 1); known = q_total; return; }
        }
    };
    // Payload q is copied by all NTHR threads, NFT 16-byte DMA pieces each,
    // into LDS buffer q % 3 (a buffer holds PBUF bytes; the tail past the
    // payload copies unused slot bytes).
    constexpr int NFT = (P::BYTES + 16 * NTHR - 1) / (16 * NTHR);
    constexpr int PBUF = NFT * 16 * NTHR;
    static_assert(PBUF <= KDA_RING_SLOT_BYTES, "slot smaller than the DMA footprint");
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const unsigned lds0 = lds_addr(lds) + wu * 64 * 16;
    auto dma = [&](int q) {
        const unsigned char *src = ring + (size_t)(q % KDA_RING) * KDA_RING_SLOT_BYTES + tid * 16;
        const unsigned dst = lds0 + (unsigned)(q % 3) * PBUF;
#pragma unroll
        for (int j = 0; j < NFT; ++j) lds_dma16(src + j * NTHR * 16, dst + j * NTHR * 16);
    };
    int chain = role.team, c = 0, nch = 0;
    ChainInfo ci{};
    f32x4 S[MT];
    size_t hbase = 0;
    bool started = false;
    auto store_hT = [&]() {
        if (computes && args.h_T) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<f32x4 *>(args.h_T + hbase + 16 * mt + 4 * lq) = S[mt];
        }
    };
    auto open_chain = [&]() {
        ci = chain_info(args, chain);
        nch = (ci.len + CH - 1) / CH;
        c = 0;
        hbase = (((size_t)ci.seq * args.H + ci.head) * DV + v0 + ln) * DK;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (args.h0 && computes) S[mt] = *reinterpret_cast<const f32x4 *>(args.h0 + hbase + 16 * mt + 4 * lq);
            else S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        vm_wait<0>();   // the state is never a pending load inside the chunk loop
    };

    // Output rows of the previous chunk, stored one step late so that the
    // stores are older than the next DMA and never delay the payload wait.
    f32x4 Op = {0.f, 0.f, 0.f, 0.f};
    size_t op_base = 0;
    int op_rem = 0;
    const size_t o_row = (size_t)args.H * DV;
    auto flush_o = [&]() {
        if (computes) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lq + i < op_rem) store_act<BF16>(args.o, op_base + (4 * lq + i) * o_row, Op[i]);
        }
        op_rem = 0;
    };

    // One chunk q, computed from LDS buffer q % 3.  Payload q+2 is requested
    // at the top; payload q+1 (requested one step earlier) is waited for at
    // the bottom, before the barrier that publishes it.
    auto step = [&](int q) {
        // chain bookkeeping (zero-length chains: h_T = h0)
        while (!started || c >= nch) {
            if (started) { store_hT(); chain += args.n_teams; }
            started = true;
            open_chain();
            if (nch == 0) c = 1;
        }
        const size_t tok0 = ci.bos + (size_t)c * CH;
        const int rem = min(CH, ci.len - c * CH);
        const bool ahead = q + 2 < q_total;
        if (ahead) ensure_ready(q + 2);
        flush_o();
        if (ahead) dma(q + 2);
        if (computes) {
            const unsigned char *pl = lds + (q % 3) * PBUF;
            // R1: W = k~ S, Qs = q~ S ; then decay the state in place
            f32x4 W = {0.f, 0.f, 0.f, 0.f}, Qs = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BF16) {
#pragma unroll
                for (int s = 0; s < DK / 32; ++s) {
                    bf16x8 b;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        b[i] = static_cast<__bf16>(S[2 * s][i]);
                        b[4 + i] = static_cast<__bf16>(S[2 * s + 1][i]);
                    }
                    const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(pl + P::KD + (s * 64 + lane) * 16);
                    const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(pl + P::QD + (s * 64 + lane) * 16);
                    W = mfma_bf16(ak, b, W);
                    Qs = mfma_bf16(aq, b, Qs);
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 ak = *reinterpret_cast<const f32x4 *>(pl + P::KD + (mt * 64 + lane) * 16);
                    const f32x4 aq = *reinterpret_cast<const f32x4 *>(pl + P::QD + (mt * 64 + lane) * 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        W = mfma_f32(ak[i], S[mt][i], W);
                        Qs = mfma_f32(aq[i], S[mt][i], Qs);
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 e = *reinterpret_cast<const f32x4 *>(pl + P::EG + (16 * mt + 4 * lq) * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[mt][i] *= e[i];
            }
            // R2: u = beta (v - W)
            const f32x4 beta = *reinterpret_cast<const f32x4 *>(pl + P::BETA + lq * 16);
            f32x4 vv;
            if constexpr (BF16) {
                const bf16x4 v4 = *reinterpret_cast<const bf16x4 *>(pl + P::V + (vt * 64 + lane) * 8);
#pragma unroll
                for (int i = 0; i < 4; ++i) vv[i] = static_cast<float>(v4[i]);
            } else {
                vv = *reinterpret_cast<const f32x4 *>(pl + P::V + (vt * 64 + lane) * 16);
            }
            f32x4 u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = beta[i] * (vv[i] - W[i]);
            // R3: U = INV u ; R4: O = Qs + Mqk U ; R5: S += k^r^T U
            f32x4 U = {0.f, 0.f, 0.f, 0.f}, O;
            if constexpr (BF16) {
                const bf16x8 inv = *reinterpret_cast<const bf16x8 *>(pl + P::INV + lane * 16);
                const bf16x8 mqk = *reinterpret_cast<const bf16x8 *>(pl + P::MQK + lane * 16);
                bf16x4 ih, il, mh, ml;
#pragma unroll
                for (int i = 0; i < 4; ++i) { ih[i] = inv[i]; il[i] = inv[4 + i]; mh[i] = mqk[i]; ml[i] = mqk[4 + i]; }
                const bf16x8 bu = split_hilo(u);
                U = mfma_bf16(dup4(ih), bu, U);
                U = mfma_bf16(dup4(il), bu, U);
                const bf16x8 bU = split_hilo(U);
                O = mfma_bf16(dup4(mh), bU, Qs);
                O = mfma_bf16(dup4(ml), bU, O);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x4 kr4 = *reinterpret_cast<const bf16x4 *>(pl + P::KR + (mt * 64 + lane) * 8);
                    S[mt] = mfma_bf16(dup4(kr4), bU, S[mt]);
                }
            } else {
                const f32x4 inv = *reinterpret_cast<const f32x4 *>(pl + P::INV + lane * 16);
                const f32x4 mqk = *reinterpret_cast<const f32x4 *>(pl + P::MQK + lane * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) U = mfma_f32(inv[i], u[i], U);
                O = Qs;
#pragma unroll
                for (int i = 0; i < 4; ++i) O = mfma_f32(mqk[i], U[i], O);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 kr4 = *reinterpret_cast<const f32x4 *>(pl + P::KR + (mt * 64 + lane) * 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[mt] = mfma_f32(kr4[i], U[i], S[mt]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Op[i] = args.scale * O[i];
            op_base = (tok0 * args.H + ci.head) * DV + v0 + ln;
            op_rem = rem;
        }
        if (ahead) vm_wait<NFT>();    // payload q+1 has landed (only q+2 may still fly)
        else vm_wait<0>();
        lds_barrier();
        if (q + 1 < q_total && tid == 0) add_flag(&used[(q + 1) % KDA_RING], 1);
        ++c;
    };

    if (q_total > 0) {
        ensure_ready(0);
        dma(0);
        if (q_total > 1) {
            ensure_ready(1);
            dma(1);
            vm_wait<NFT>();
        } else {
            vm_wait<0>();
        }
        lds_barrier();
        if (tid == 0) add_flag(&used[0], 1);
    }
    for (int q = 0; q < q_total; ++q) step(q);
    flush_o();
    // final state of the last open chain, then any trailing zero-length chains
    if (started) store_hT();
    for (chain = started ? chain + args.n_teams : role.team; chain < n_chains; chain += args.n_teams) {
        open_chain();
        store_hT();
    }
}

template <bool BF16, int DK, int DV, int BDV>
static hipError_t launch_one(ChunkArgs a, hipStream_t stream)
{
    constexpr int NS = DV / BDV;
    constexpr int TS = NS + KDA_PRODUCER_WGS;
    const int n_chains = a.n_seq * a.H;
    if (n_chains == 0) return hipSuccess;
    int dev = 0, n_cu = 0, occ = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, chunk_fwd_kernel<BF16, DK, DV, BDV>, NTHR, 0);
    if (e != hipSuccess) return e;
    // every workgroup of the grid must be resident at once (teams wait on each other)
    const int cap_wgs = n_cu * (occ < 1 ? 1 : occ);
    int teams_per_xcd = cap_wgs / (8 * TS);
    if (teams_per_xcd < 1) return hipErrorInvalidConfiguration;
    const int need_per_xcd = (n_chains + 7) / 8;
    if (teams_per_xcd > need_per_xcd) teams_per_xcd = need_per_xcd;
    int n_teams = 8 * teams_per_xcd;
    if (n_teams > n_chains) n_teams = n_chains;
    if (n_teams > KDA_MAX_TEAMS) n_teams = KDA_MAX_TEAMS;
    a.n_teams = n_teams;
    e = hipMemsetAsync(a.flags, 0, sizeof(int) * (2 * (size_t)KDA_MAX_TEAMS * KDA_RING + 64), stream);
    if (e != hipSuccess) return e;
    const unsigned grid = 8u * TS * (unsigned)((n_teams + 7) / 8);
    hipLaunchKernelGGL((chunk_fwd_kernel<BF16, DK, DV, BDV>), dim3(grid), dim3(NTHR), 0, stream, a);
    return hipGetLastError();
}

// d_v slab width: enough consumer workgroups to cover the device, at most 64
// columns (4 compute waves) and at least 16.
static int pick_bdv(int n_chains, int dv)
{
    int bdv = dv < 64 ? dv : 64;
    while (bdv > 16 && n_chains * (dv / bdv) < 256) bdv /= 2;
    return bdv;
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int dk, int dv, hipStream_t stream)
{
    const int bdv = pick_bdv(a.n_seq * a.H, dv);
#define KDA_DISPATCH(BF, DKV, DVV)                                             \
    if (dk == DKV && dv == DVV) {                                              \
        if (bdv == 64 && DVV >= 64) return launch_one<BF, DKV, DVV, 64>(a, stream); \
        if (bdv == 32) return launch_one<BF, DKV, DVV, 32>(a, stream);         \
        return launch_one<BF, DKV, DVV, 16>(a, stream);                        \
    }
    if (dtype == 1) {
        KDA_DISPATCH(true, 128, 128)
        KDA_DISPATCH(true, 128, 64)
        KDA_DISPATCH(true, 64, 128)
        KDA_DISPATCH(true, 64, 64)
    } else {
        KDA_DISPATCH(false, 64, 128)
        KDA_DISPATCH(false, 64, 64)
    }
#undef KDA_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace kda
