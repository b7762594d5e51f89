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
// per d_v slab of BDV = 32 columns, each holding its fp32 state slab in MFMA
// accumulators for the whole walk over the sequence.  One TEAM = NS consumer
// workgroups + NP = 4 producer workgroups for one (sequence, head) chain at a
// time.  The four waves of a producer build one chunk together (producer p
// takes chunks p, p + NP, ...) and write an ~18 KiB payload, already in MFMA
// fragment order, into a ring of KDA_RING slots in device memory.  In every
// consumer two compute waves run the recurrence (and store their outputs) and
// two helper waves poll the ring and copy each payload into LDS two chunks
// ahead.
// The prep therefore runs once per chunk for all d_v slabs instead of once
// per slab.
//
// Ring protocol.  All workgroups of a team share blockIdx % 8, i.e. run on the
// same XCD and share its L2 (MI355X dispatches workgroups to its 8 XCDs round
// robin).  A producer writes the payload with ordinary stores, waits for them
// (s_waitcnt vmcnt(0): stores are acknowledged by L2), then stores the slot's
// ready flag with an L2-coherent (sc1) store.  A consumer reads the flags and
// the payload with sc1 loads (LDS DMA), which read L2 and never a stale L1
// line.  After the copy it adds 1 to the slot's use counter; a producer reuses
// a slot once all NS consumers have copied it.  No device-scope cache
// write-back or L2 invalidation is needed.  Every wait is bounded; on timeout
// the kernel sets an error word and stops waiting, so it always terminates.
// All workgroups of the grid must be resident at once; the host sizes the grid
// from the occupancy query.
//
// Overflow-safe L / Mqk.  The factored form <k_i e^{G_i}, k_j e^{-G_j}> leaves
// the fp32 range once a channel decays by more than ~88 nats inside a chunk.
// A chunk in which every channel's total decay is at most 100 in log2 units
// ("mild") uses one reference at the chunk end:
//   rows k_i 2^{g_C - g_i} (<= 2^100), columns k^r_j = k_j 2^{g_j - g_C} (<= 1).
// Other chunks use row blocks of BR tokens: for rows in block b the reference
// is the cumulative decay g' at the end of block b-1, with each token's decay
// clipped at CLIP (e^g floored at 2^-CLIP):
//   rows k_i 2^{g'_ref - g'_i} (<= 1),  columns k_j 2^{g'_j - g'_ref}
//   (<= 2^{BR CLIP} inside block b, <= 1 before it),
// one MFMA pass per row block.  Pairs whose true decay gap exceeds CLIP
// (log2) are then computed as at most 2^-CLIP instead of their (smaller) true
// value; everything else is exact.  The fp32 build takes four 4-token blocks
// with CLIP = 24 (an error below fp32 rounding of the O(1) entries); the bf16
// build, whose L and Mqk operands are rounded to bf16 (2^-9 relative), takes
// two 8-token blocks with CLIP = 12.
// The state-side operands (k~, q~, k^r) and the state decay use the unclipped
// gates; all their factors are <= 1, so underflow only drops negligible terms.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int CH = 16;              // chunk length (tokens)
constexpr int NTHR = 256;           // threads per workgroup (4 waves), both roles
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
                 : "=&s"(saved) : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {       // at most N vector-memory ops of this wave in flight
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}
// At most n (wave-uniform, 0 .. 4) vector-memory ops of this wave in flight.
__device__ __forceinline__ void vm_wait_le(int n) {
    switch (n) {
    case 4: vm_wait<4>(); break;
    case 3: vm_wait<3>(); break;
    case 2: vm_wait<2>(); break;
    case 1: vm_wait<1>(); break;
    default: vm_wait<0>(); break;
    }
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
//       INV/MQK: lane 8 B = X[ln][4lq .. 4lq+3].
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
    static constexpr int MQK = INV + 64 * KRB;
    static constexpr int BETA = MQK + 64 * KRB;
    static constexpr int EG = BETA + 64;
    static constexpr int V = (EG + DK * 4 + 1023) / 1024 * 1024;   // v (1 KiB aligned): fragment vt,
                                                                   // lane: rows 4lq..4lq+3 of column 16vt+ln
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

// A operand pairing with a [hi | lo] B operand: the row values repeated in
// both K halves.
__device__ __forceinline__ bf16x8 dup4(bf16x4 a) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = a[i]; }
    return r;
}
// 4x4 transpose inside each quad of lanes (two DPP butterflies): lane j of the
// quad gets element j of each quad lane, i.e. out[r] = lane r's x[j].
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int j) {
    f32x4 a, b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float y = dpp_f<0xB1>(x[r ^ 1]);     // lane j ^ 1
        a[r] = ((r ^ j) & 1) == 0 ? x[r] : y;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float y = dpp_f<0x4E>(a[r ^ 2]);     // lane j ^ 2
        b[r] = ((r ^ j) & 2) == 0 ? a[r] : y;
    }
    return b;
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
// Workgroups are dispatched to the 8 XCDs round robin (blockIdx % 8); within
// an XCD the first `pair_half` workgroups (one per CU) take every CU once and
// workgroup y + pair_half then lands on the same CU as workgroup y.  With
// pair_half > 0 a team occupies ceil(TS/2) CUs: the older workgroup of each
// CU takes members 0, 1, ... (the consumers first), the younger one the
// matching later member (the producers), so consumers share their CU with a
// producer of their own team and win instruction arbitration against it.
// With pair_half == 0 (one workgroup per CU) members are consecutive.
__device__ __forceinline__ Role role_of(int NS, int NP, int n_teams, int pair_half, int teams_per_xcd) {
    const int TS = NS + NP;
    const int x = blockIdx.x % 8, y = blockIdx.x / 8;
    int tx, member;
    if (pair_half > 0) {
        const int cpt = (TS + 1) / 2;                 // CUs per team
        const int h = y >= pair_half ? 1 : 0, yy = y - h * pair_half;
        tx = yy / cpt;
        member = yy - tx * cpt + h * cpt;
    } else {
        tx = y / TS;
        member = y - tx * TS;
    }
    Role r;
    r.team = tx * 8 + x;
    r.member = member;
    if (member >= TS || tx >= teams_per_xcd || r.team >= n_teams) r.team = -1;
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
// A producer workgroup builds whole chunks with all four waves.  Lane
// (wave w, lane 16 r + t) holds token t of the chunk and the 16-byte unit
// u = 4 w + r of its k, q and g_raw rows, i.e. UC = 16 / element-size
// channels [UC u, UC u + UC).  A DPP row (16 lanes) thus holds one channel
// unit for all 16 tokens: the chunk-local cumulative gate is a 16-lane scan,
// a lane's k~ / q~ values are exactly one 16-byte MFMA fragment of the payload
// (the consumer's state tiles use the matching channel order, tile_chan()),
// and a wave's registers are directly the A and B operands of its share of
// the L / Mqk contractions (UC * 4 channels per wave).

// Channel held by row 4 lq + i of the consumer's state tile mt (and by the
// same rows of the k^r fragments and of e^{G_C}).  For bf16 the 8 K slots a
// lane feeds to a 16x16x32 MFMA are then 8 contiguous channels.
template <bool BF16>
__device__ __forceinline__ int tile_chan(int mt, int lq, int i) {
    if constexpr (BF16) return 32 * (mt >> 1) + 8 * lq + 4 * (mt & 1) + i;
    else return 16 * mt + 4 * lq + i;
}

// Producer LDS: v and k^r transposed to [column / channel][token] (a
// consumer fragment of 4 tokens of one column is then one contiguous read;
// rows padded so the writers of neighbouring channels use different banks),
// the per-wave partial 16x16 sums (L and Mqk^T) and beta.
template <bool BF16, int DK, int DV>
struct PG {
    static constexpr int ES = BF16 ? 2 : 4;
    static constexpr int UC = 16 / ES;              // elements per 16-byte unit
    static constexpr int NU = DK / UC;              // k / q / g_raw units per token
    static constexpr int NVU = DV / UC;             // v units per token
    static constexpr int NWU = NU / 4;              // waves holding channel units
    static constexpr int NVP = 16 * NVU / 64;       // v units per chunk / 64
    static constexpr int NVL = (NVP + 3) / 4;       // v units per lane
    static constexpr int TP = 16 * ES + (BF16 ? 8 : 16);   // bytes per transposed row (16 tokens + pad)
    static constexpr int VT = 0;                    // v^T: [DV][16 tokens]
    static constexpr int KRT = VT + DV * TP;        // k^r^T: [DK][16 tokens]
    static constexpr int PART = KRT + DK * TP;
    static constexpr int SBETA = PART + NWU * 2 * 64 * 16;
    static constexpr int BYTES = SBETA + CH * 4;
    static_assert(NU % 4 == 0 && NU <= 16, "4..16 channel units");
    static_assert(NVP >= 1 && (16 * NVU) % 64 == 0, "v units");
};

// The producer wave that forms INV (a serial chain of small MFMA products).
// Its SIMD partner on the CU is a consumer helper wave, which mostly waits, so
// the chain is not starved by the consumer's higher-priority compute.
constexpr int PROD_INV_WAVE = 3;

// One chunk's inputs as one producer lane holds them: its k, q, g_raw units
// (wave w < NWU), v units 64 m + lane for m = w, w + 4, ... (< NVP), and, in
// wave PROD_INV_WAVE, beta_raw of token `lane`.
template <bool BF16, int DK, int DV>
struct PIn {
    uint4 k, q, a;
    uint4 v[PG<BF16, DK, DV>::NVL];
    typename Elem<BF16>::T b;   // raw bits: converted only where used
};

// DPP (dpp_f of kda_device.hpp): row_shr n gives x of the lane n below in the
// same 16-lane row (0 past the row start); row_newbcast n broadcasts lane n.
__device__ __forceinline__ float scan16(float x) {   // inclusive prefix sum over the row's 16 tokens
    x += dpp_f<0x111>(x);
    x += dpp_f<0x112>(x);
    x += dpp_f<0x114>(x);
    x += dpp_f<0x118>(x);
    return x;
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) { return dpp_f<0x150 + N>(x); }

// A team's chunk sequence (its chains one after the other, in chain order).
struct Cursor {
    int chain, q_base, nch;
    ChainInfo ci;
};
__device__ __forceinline__ void cursor_seek(Cursor &c, int q, const ChunkArgs &a, int n_teams) {
    while (q >= c.q_base + c.nch) {
        c.q_base += c.nch;
        c.chain += n_teams;
        c.ci = chain_info(a, c.chain);
        c.nch = (c.ci.len + CH - 1) / CH;
    }
}

// Issue the loads of team chunk q's inputs into `in`.  Rows past the chunk's
// live tokens repeat the last live row (always in bounds); their values are
// masked where used.  The loads sit in no lane-divergent branch, so nothing
// waits for them before their use one chunk later.
template <bool BF16, int DK, int DV>
__device__ __forceinline__ void prod_load(PIn<BF16, DK, DV> &in, const Cursor &c, int q, const ChunkArgs &a,
                                          int w, int lane) {
    using G = PG<BF16, DK, DV>;
    const int cc = q - c.q_base;
    const size_t tok0 = c.ci.bos + (size_t)cc * CH;
    const int last = min(CH, c.ci.len - cc * CH) - 1;
    const size_t H = a.H, h = c.ci.head;
    if (w < G::NWU) {
        const int t = lane & 15, u = 4 * w + (lane >> 4);
        const size_t off = (((tok0 + min(t, last)) * H + h) * DK) * G::ES + u * 16;
        in.k = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.k) + off);
        in.q = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) + off);
        in.a = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.g_raw) + off);
    }
#pragma unroll
    for (int j = 0; j < G::NVL; ++j) {
        const int m = w + 4 * j;
        if (m < G::NVP) {
            const int p = 64 * m + lane, tv = p / G::NVU, vu = p - tv * G::NVU;
            const size_t off = (((tok0 + min(tv, last)) * H + h) * DV) * G::ES + vu * 16;
            in.v[j] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.v) + off);
        }
    }
    if (w == PROD_INV_WAVE) in.b = static_cast<const typename Elem<BF16>::T *>(a.beta_raw)[(tok0 + min(lane, last)) * H + h];
}

// 8 values as one bf16 MFMA operand (RNE).
__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}
__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}
__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}
__device__ __forceinline__ f32x4 contract4(const float (&X)[4], const float (&Y)[4], f32x4 acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma_f32(X[i], Y[i], acc);
    return acc;
}

// 16x16x16 product in C layout without any data movement: given XT = C layout
// of X^T (lane (lq, ln) element i = X[ln][4lq+i], which is the A operand's
// element) and Y in C layout (the B operand's element), return X Y in C layout.
__device__ __forceinline__ f32x4 prod16(f32x4 XT, f32x4 Y) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma_f32(XT[i], Y[i], acc);   // fp32 MFMA, K = 4 per step
    return acc;
}
// The same product from single-bf16 operands (upper K half zero): one MFMA.
__device__ __forceinline__ f32x4 prod16b(f32x4 XT, f32x4 Y) {
    bf16x8 a = {}, b = {};
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = static_cast<__bf16>(XT[i]); b[i] = static_cast<__bf16>(Y[i]); }
    return mfma_bf16(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
}
__device__ __forceinline__ f32x4 plus_eye(f32x4 X, int ln, int lq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) X[i] += (4 * lq + i == ln) ? 1.f : 0.f;
    return X;
}

template <bool BF16>
__device__ __forceinline__ void unpack16(uint4 v, float (&x)[16 / (BF16 ? 2 : 4)]) {
    if constexpr (BF16) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __builtin_bit_cast(float, wv[j] << 16);
            x[2 * j + 1] = __builtin_bit_cast(float, wv[j] & 0xffff0000u);
        }
    } else {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __builtin_bit_cast(float, wv[j]);
    }
}
template <bool BF16>
__device__ __forceinline__ void pack16(void *p, const float (&x)[16 / (BF16 ? 2 : 4)]) {
    if constexpr (BF16) {
        uint4 v;
        v.x = pack_bf16x2(x[0], x[1]);
        v.y = pack_bf16x2(x[2], x[3]);
        v.z = pack_bf16x2(x[4], x[5]);
        v.w = pack_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4 *>(p) = v;
    } else {
        *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
    }
}

// ============================================================== the kernel
__device__ __forceinline__ void lds_barrier() {   // LDS-only barrier: global ops stay in flight
    lds_done();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// SNAP: also store the state entering every chunk to args.h_chunks.
template <bool BF16, int DK, int DV, int BDV, bool SNAP>
__global__ __launch_bounds__(NTHR, 2) void chunk_fwd_kernel(ChunkArgs args)
{
    using P = PL<BF16, DK, DV>;
    constexpr int NS = DV / BDV;
    constexpr int NCW = BDV / 16;          // compute waves of a consumer workgroup
    constexpr int MT = DK / 16;
    constexpr int NP = KDA_PRODUCER_WGS;
    static_assert(NCW == 2, "consumer slab of 32 columns: two compute and two helper waves");
    static_assert(KDA_RING <= 32, "one lane per ring slot when polling; ready and used in their own lines");

    // Consumers copy, per payload, the blocks (1 KiB each) up to v and then their
    // slab's v blocks only, compactly into one of NBUF LDS buffers of CBUF bytes.
    constexpr int FB = 64 * 4 * P::ES;            // bytes per v fragment
    constexpr int VB0 = P::V / 1024;
    constexpr int NSB = ((BDV / 16) * FB + 1023) / 1024;
    constexpr int NCB = VB0 + NSB;
    constexpr int CBUF = NCB * 1024;
    constexpr int NBUF = 4;                      // compute q, copies of q+1 .. q+3 in flight
    // LDS: producers use their input buffers and scratch; consumers the payload
    // buffers and three poll spots of KDA_RING flags.
    constexpr int PROD_BYTES = PG<BF16, DK, DV>::BYTES;
    constexpr int CONS_BYTES = NBUF * CBUF + 3 * 4 * KDA_RING;
    constexpr int LDS_BYTES = PROD_BYTES > CONS_BYTES ? PROD_BYTES : CONS_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    const Role role = role_of(NS, NP, args.n_teams, args.pair_half, args.teams_per_xcd);
    if (role.team < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;
    constexpr int SLOT = P::BYTES;               // ring slot (whole 1 KiB blocks)
    static_assert(SLOT <= KDA_RING_SLOT_BYTES, "slot larger than the workspace's");
    unsigned char *ring = args.ring + (size_t)role.team * KDA_RING * SLOT;
    int *ready = args.flags + (size_t)role.team * KDA_TEAM_FLAG_INTS;
    int *used = ready + 32;
    int *err = args.err;
    const int n_chains = args.n_seq * args.H;

    if (role.member >= NS) {
        // ======================================================= producer
        using G = PG<BF16, DK, DV>;
        constexpr int UC = G::UC;
        const int wu = __builtin_amdgcn_readfirstlane(w);
        const int p = role.member - NS;                 // chunks p, p + NP, p + 2 NP, ... of the team
        const int t = ln, r = lq, u = 4 * wu + r;       // token, channel unit
        const bool has_unit = wu < G::NWU;
        float *sbeta = reinterpret_cast<float *>(lds + G::SBETA);
        int q_total = 0;
        for (int chain = role.team; chain < n_chains; chain += args.n_teams)
            q_total += (chain_info(args, chain).len + CH - 1) / CH;
        if (p >= q_total) return;
        Cursor cp;
        cp.chain = role.team;
        cp.q_base = 0;
        cp.ci = chain_info(args, cp.chain);
        cp.nch = (cp.ci.len + CH - 1) / CH;
        cursor_seek(cp, p, args, args.n_teams);         // the chain holding this producer's first chunk
        Cursor cd = cp;                                 // the chunk being loaded, one step ahead
        PIn<BF16, DK, DV> cur, nxt;
        prod_load<BF16, DK, DV>(cur, cp, p, args, wu, lane);
        // `cur` is never a pending load inside the loop (there it is a copy of
        // `nxt` made after the drain); without this wait the compiler would
        // wait inside the loop for the next chunk's loads before using `cur`
        vm_wait<0>();
        int cur_chain = -1;
        float A_exp = 0.f, dtl[UC];
        for (int it = 0;; ++it) {
            const int q = p + it * NP;
            if (q >= q_total) break;
            cursor_seek(cp, q, args, args.n_teams);
            const int rem = min(CH, cp.ci.len - (q - cp.q_base) * CH);
            if (cp.chain != cur_chain) {
                cur_chain = cp.chain;
                A_exp = expf(args.A_log[cp.ci.head]);
#pragma unroll
                for (int c = 0; c < UC; ++c)
                    dtl[c] = has_unit ? args.dt_bias[(size_t)cp.ci.head * DK + UC * u + c] * kLog2e : 0.f;
            }
            const int s = q % KDA_RING;
            unsigned char *slot = ring + (size_t)s * SLOT;
            // slot free?  (polled before this step's loads are issued, so the poll's
            // wait covers nothing else; spinning on scalar loads instead would
            // starve the instruction fetch of neighbouring compute units)
            if (q >= KDA_RING) wait_geq(&used[s], NS * (q / KDA_RING), err);
            // the producer's next chunk loads while this one is built (the loads
            // have had a whole step when the stores below are drained)
            const int qn = q + NP;
            if (qn < q_total) {
                cursor_seek(cd, qn, args, args.n_teams);
                prod_load<BF16, DK, DV>(nxt, cd, qn, args, wu, lane);
            }
            // v to LDS as [column][token] (padding tokens zero) for the fragment writers
            using E = typename Elem<BF16>::T;
#pragma unroll
            for (int j = 0; j < G::NVL; ++j) {
                const int m = wu + 4 * j;
                if (m < G::NVP) {
                    const int pv = 64 * m + lane, tv = pv / G::NVU, vu = pv - tv * G::NVU;
                    const uint4 x = cur.v[j];
                    const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int e = 0; e < G::UC; ++e) {
                        E val;
                        if constexpr (BF16) val = (E)(wv[e >> 1] >> (16 * (e & 1)));
                        else val = __builtin_bit_cast(float, wv[e]);
                        *reinterpret_cast<E *>(lds + G::VT + (G::UC * vu + e) * G::TP + tv * G::ES) =
                            tv < rem ? val : E(0);
                    }
                }
            }

            if (has_unit) {
                // ---- gate and its chunk-local cumulative sum (log2 units), per channel
                float kf[UC], qf[UC], af[UC], gv[UC], Gm[UC], GC[UC];
                unpack16<BF16>(cur.k, kf);
                unpack16<BF16>(cur.q, qf);
                unpack16<BF16>(cur.a, af);
                const bool live = t < rem;
                bool deep = false;
#pragma unroll
                for (int c = 0; c < UC; ++c) {
                    kf[c] = live ? kf[c] : 0.f;
                    qf[c] = live ? qf[c] : 0.f;
                    const float y = __builtin_fmaf(af[c], kLog2e, dtl[c]);
                    const float sp2 = y > 20.0f * kLog2e ? y : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(y));
                    gv[c] = live ? -A_exp * sp2 : 0.f;    // padded tokens do not decay
                    Gm[c] = scan16(gv[c]);
                    GC[c] = row_bcast<15>(Gm[c]);
                    deep |= GC[c] < -100.f;
                }
                // ---- k~ = k 2^G, q~ = q 2^G (payload fragments), k^r = k 2^{G_C - G}, e^{G_C}
                float kd[UC], qd[UC], kr[UC], e1[UC];
#pragma unroll
                for (int c = 0; c < UC; ++c) {
                    e1[c] = __builtin_amdgcn_exp2f(Gm[c]);
                    kd[c] = kf[c] * e1[c];
                    qd[c] = qf[c] * e1[c];
                    kr[c] = kf[c] * __builtin_amdgcn_exp2f(GC[c] - Gm[c]);
                }
                pack16<BF16>(slot + P::KD + tid * 16, kd);
                pack16<BF16>(slot + P::QD + tid * 16, qd);
#pragma unroll
                for (int c = 0; c < UC; ++c)
                    *reinterpret_cast<E *>(lds + G::KRT + (UC * u + c) * G::TP + t * G::ES) = to_elem<BF16>(kr[c]);
                if (t == CH - 1) {
                    float *eg = reinterpret_cast<float *>(slot + P::EG);
                    if constexpr (BF16) {
                        *reinterpret_cast<f32x4 *>(eg + 16 * (2 * wu) + 4 * r) = f32x4{e1[0], e1[1], e1[2], e1[3]};
                        *reinterpret_cast<f32x4 *>(eg + 16 * (2 * wu + 1) + 4 * r) = f32x4{e1[4], e1[5], e1[6], e1[7]};
                    } else {
                        *reinterpret_cast<f32x4 *>(eg + 16 * wu + 4 * r) = f32x4{e1[0], e1[1], e1[2], e1[3]};
                    }
                }
                // ---- this wave's share of L (rows i), L^T and Mqk^T over its UC*4 channels
                f32x4 pL = {0.f, 0.f, 0.f, 0.f}, pMT = pL;
                if (__ballot(deep) == 0) {
                    // mild: one reference at the chunk end, rows k 2^{G - G_C} (<= 2^100), columns k^r (<= 1)
                    float R[UC], Rq[UC];
#pragma unroll
                    for (int c = 0; c < UC; ++c) {
                        const float f = __builtin_amdgcn_exp2f(Gm[c] - GC[c]);
                        R[c] = kf[c] * f;
                        Rq[c] = qf[c] * f;
                    }
                    if constexpr (BF16) {
                        // one MFMA over the wave's 32 channels (k slot e of lane (lq, ln) = channel e of unit lq)
                        const bf16x8 bC = pack8(kr);
                        pL = mfma_bf16(pack8(R), bC, pL);
                        pMT = mfma_bf16(bC, pack8(Rq), pMT);
                    } else {
                        pL = contract4(R, kr, pL);
                        pMT = contract4(kr, Rq, pMT);
                    }
                } else {
                    // strong: row blocks of BR tokens, each token's decay clipped at 2^-CLIP, so that a
                    // column factor inside its block stays <= 2^(BR CLIP) <= 2^96; block b's reference is
                    // the clipped cumulative decay at the end of block b-1.  The bf16 build rounds the
                    // entries to bf16 anyway, so it clips at 2^-12 (two 8-token blocks); fp32 clips at
                    // 2^-24 (four 4-token blocks).
                    constexpr int NB = BF16 ? 2 : 4, BR = CH / NB;
                    constexpr float CLIP = BF16 ? 12.0f : 24.0f;
                    float Gp[UC], Bf[NB][UC], R[UC], Rq[UC];
#pragma unroll
                    for (int c = 0; c < UC; ++c) {
                        Gp[c] = scan16(fmaxf(gv[c], -CLIP));
                        Bf[0][c] = 0.f;
                        if constexpr (NB == 2) {
                            Bf[1][c] = row_bcast<7>(Gp[c]);
                        } else {
                            Bf[1][c] = row_bcast<3>(Gp[c]);
                            Bf[2][c] = row_bcast<7>(Gp[c]);
                            Bf[3][c] = row_bcast<11>(Gp[c]);
                        }
                        float ref = Bf[0][c];
#pragma unroll
                        for (int bb = 1; bb < NB; ++bb) ref = t >= BR * bb ? Bf[bb][c] : ref;
                        const float f = __builtin_amdgcn_exp2f(Gp[c] - ref);     // <= 1
                        R[c] = kf[c] * f;
                        Rq[c] = qf[c] * f;
                    }
                    [[maybe_unused]] bf16x8 bR, bRq;
                    if constexpr (BF16) { bR = pack8(R); bRq = pack8(Rq); }
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        float C[UC];
#pragma unroll
                        for (int c = 0; c < UC; ++c)
                            C[c] = t < BR * (bb + 1) ? kf[c] * __builtin_amdgcn_exp2f(Bf[bb][c] - Gp[c]) : 0.f;
                        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                        f32x4 Lb, MTb;
                        if constexpr (BF16) {
                            const bf16x8 bC = pack8(C);
                            Lb = mfma_bf16(bR, bC, z);
                            MTb = mfma_bf16(bC, bRq, z);
                        } else {
                            Lb = contract4(R, C, z);
                            MTb = contract4(C, Rq, z);
                        }
                        // keep the rows (of L and Mqk) that lie in block bb: C-layout rows 4r .. 4r+3
                        // of L, column t of Mqk^T
                        if ((4 * r) / BR == bb) pL = Lb;
                        if (t / BR == bb) pMT = MTb;
                    }
                }
                f32x4 *pp = reinterpret_cast<f32x4 *>(lds + G::PART) + (wu * 2) * 64 + lane;
                pp[0] = pL;
                pp[64] = pMT;
            }
            if (wu == PROD_INV_WAVE && lane < CH) {
                float bv;
                if constexpr (BF16) bv = bf16_to_f32(cur.b);
                else bv = cur.b;
                sbeta[lane] = lane < rem ? sigmoid_f(bv) : 0.f;
            }
            lds_barrier();

            if (wu == PROD_INV_WAVE) {
                // ---- L, L^T (C layout; L^T read transposed from the L sums), masks and beta;
                // INV by Neumann squaring in transposed pairs
                f32x4 L = {0.f, 0.f, 0.f, 0.f}, LT = L, MQ = L;
                const f32x4 *pp = reinterpret_cast<const f32x4 *>(lds + G::PART) + lane;
                const float *pf = reinterpret_cast<const float *>(lds + G::PART);
#pragma unroll
                for (int ww = 0; ww < G::NWU; ++ww) {
                    L += pp[ww * 128];
                    MQ += pp[ww * 128 + 64];
#pragma unroll
                    for (int i = 0; i < 4; ++i)   // L[ln][4lq+i]: lane 16(ln/4) + 4lq + i, element ln % 4
                        LT[i] += pf[(ww * 128 + 16 * (ln >> 2) + 4 * lq + i) * 4 + (ln & 3)];
                }
                const f32x4 brow = *reinterpret_cast<const f32x4 *>(sbeta + 4 * lq);
                const float bcol = sbeta[ln];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * lq + i;
                    L[i] = row > ln ? -brow[i] * L[i] : 0.f;      // L[row][ln], strictly lower
                    LT[i] = ln > row ? -bcol * LT[i] : 0.f;       // L[ln][row]
                    MQ[i] = ln >= row ? MQ[i] : 0.f;              // Mqk[ln][row], lower incl. diagonal
                }
                // C-layout operands feed the MFMAs directly: fp32 16x16x4 MFMAs for the
                // fp32 build; single-bf16 products for the bf16 build, whose INV is
                // rounded to bf16 for the payload anyway
                auto pr = [](f32x4 XT, f32x4 Y) { return BF16 ? prod16b(XT, Y) : prod16(XT, Y); };
                const f32x4 L2 = pr(LT, L), L2T = pr(L, LT);
                const f32x4 L4 = pr(L2T, L2), L4T = pr(L2, L2T);
                const f32x4 L8 = pr(L4T, L4);
                // A^T = ((I + L)(I + L^2))^T,  B = (I + L^4)(I + L^8),  INV^T = B^T A^T
                const f32x4 AT = pr(plus_eye(L2, ln, lq), plus_eye(LT, ln, lq));
                const f32x4 Bm = pr(plus_eye(L4T, ln, lq), plus_eye(L8, ln, lq));
                const f32x4 IT = pr(Bm, AT);
                if constexpr (BF16) {
                    *reinterpret_cast<bf16x4 *>(slot + P::INV + lane * 8) = pack4(IT);
                    *reinterpret_cast<bf16x4 *>(slot + P::MQK + lane * 8) = pack4(MQ);
                } else {
                    *reinterpret_cast<f32x4 *>(slot + P::INV + lane * 16) = IT;
                    *reinterpret_cast<f32x4 *>(slot + P::MQK + lane * 16) = MQ;
                }
                if (lane < CH) reinterpret_cast<float *>(slot + P::BETA)[lane] = sbeta[lane];
            } else {
                // ---- k^r fragments (from the staging area) and v fragments (from the inputs)
                constexpr int NKR = (DK / 16) * 64, NVF = (DV / 16) * 64;
                constexpr int PER = BF16 ? 2 : 1;       // fragment lanes per thread: 16-byte stores
                const int ft = wu < PROD_INV_WAVE ? tid : tid - 64;   // threads of the other three waves
                for (int idx0 = ft * PER; idx0 < NKR + NVF; idx0 += (NTHR - 64) * PER) {
                    using Piece = typename std::conditional<BF16, uint2, f32x4>::type;
                    Piece v[PER];
                    int dst = 0;
#pragma unroll
                    for (int e = 0; e < PER; ++e) {
                        const int idx = idx0 + e;
                        const int l2 = idx & 63, lq2 = l2 >> 4, ln2 = l2 & 15;
                        int src;   // 4 tokens of one channel / column: 4 * ES contiguous bytes
                        if (idx < NKR) {
                            const int mt = idx >> 6;
                            src = G::KRT + tile_chan<BF16>(mt, ln2 >> 2, ln2 & 3) * G::TP + 4 * lq2 * G::ES;
                            if (e == 0) dst = P::KR + (mt * 64 + l2) * P::KRB;
                        } else {
                            const int vt = (idx - NKR) >> 6;
                            src = G::VT + (16 * vt + ln2) * G::TP + 4 * lq2 * G::ES;
                            if (e == 0) dst = P::V + (vt * 64 + l2) * 4 * G::ES;
                        }
                        v[e] = *reinterpret_cast<const Piece *>(lds + src);
                    }
                    // consecutive fragment lanes are consecutive in the payload (NKR is even)
                    if constexpr (BF16) *reinterpret_cast<uint4 *>(slot + dst) = uint4{v[0].x, v[0].y, v[1].x, v[1].y};
                    else *reinterpret_cast<f32x4 *>(slot + dst) = v[0];
                }
            }
            stores_done();
            lds_barrier();
            if (tid == 0) st_flag(&ready[s], q + 1);
            cur = nxt;
        }
        return;
    }

    // =========================================================== consumer
    const int slab = role.member;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const bool computes = wu < NCW;
    const int v0 = slab * BDV + 16 * (computes ? wu : 0);
    const int vt = v0 >> 4;
    // The helper waves (those beyond the slab's compute waves) poll the ring and
    // copy the payloads into LDS while the compute waves work; the compute
    // waves' only memory instructions are their output stores.  (Giving the
    // compute waves a share of the copy was measured slower.)
    constexpr int NH = 4 - NCW;                   // helper waves
    constexpr int CPW = NH;                       // copying waves
    const bool copier = wu >= NCW;
    const int cw = wu - NCW;                      // index among the copying waves
    const int poller = NCW;                       // the wave that polls the ready flags
    int *pollbuf = reinterpret_cast<int *>(lds + NBUF * CBUF);   // [3][KDA_RING] ready flags
    const int SB0 = (P::V + slab * (BDV / 16) * FB) / 1024;     // first copied v block (global)
    int q_total = 0;
    for (int chain = role.team; chain < n_chains; chain += args.n_teams)
        q_total += (chain_info(args, chain).len + CH - 1) / CH;

    // Ready tracking: chunks <= known are ready (each copying wave keeps its
    // own `known`).  Every step the first copying wave copies the RING ready
    // flags into an LDS poll spot with the same LDS DMA as the payloads; the
    // answer is read two steps later, after that wave's vmcnt wait and a
    // barrier, from spot (step % 3), so the L2 round trip never stalls a step
    // and the poll costs one memory instruction per workgroup.  (A
    // compiler-visible load would also make the compiler wait for the younger
    // payload copies.)  Only a chunk still not ready by then costs a blocking
    // poll.  Flags only grow, so an old answer stays true.
    int known = -1;
    auto run_from = [&](int f, int need) {   // number of consecutive ready chunks from need
        const int cj = need + lane;
        const int fj = __shfl(f, cj % KDA_RING);
        const unsigned long long ok = __ballot(lane < KDA_RING && fj >= cj + 1);
        return (int)__builtin_ctzll(~ok);
    };
    static_assert(KDA_RING % 4 == 0, "the poll copies the flags 16 bytes per lane");
    auto poll_issue = [&](int spot) {
        if (wu == poller && lane < KDA_RING / 4) lds_dma16(ready + 4 * lane, lds_addr(pollbuf + KDA_RING * spot));
    };
    auto ensure_ready = [&](int need, int spot) {   // spot < 0: no poll answer to read
        if (need <= known) return;
        if (spot >= 0) {          // lane i checks chunk need + i in its slot directly
            const int cj = need + lane;
            const int fj = lane < KDA_RING ? pollbuf[KDA_RING * spot + cj % KDA_RING] : 0;
            const unsigned long long ok = __ballot(lane < KDA_RING && fj >= cj + 1);
            const int run = (int)__builtin_ctzll(~ok);
            if (run > 0) { known = need + run - 1; return; }
        }
        for (long n = 0;; ++n) {
            const int run = run_from(lane < KDA_RING ? ld_flag(&ready[lane]) : 0, need);
            if (run > 0) { known = need + run - 1; return; }
            // not ready yet: give up if another wait already did, else wait a little
            if (ld_flag(err) || n > SPIN_LIMIT) { st_flag(err, 1); known = q_total; return; }
            __builtin_amdgcn_s_sleep(2);
        }
    };
    // This wave's share of the copy of payload q into LDS buffer q % NBUF:
    // copy blocks j = cw, cw + CPW, ... < NCB (lane i moves bytes 16 i .. 16 i + 15);
    // block j < VB0 is payload block j, the others this slab's v blocks.
    auto dma = [&](int q) {
        const unsigned char *src = ring + (size_t)(q % KDA_RING) * SLOT + lane * 16;
        const unsigned dst = lds_addr(lds) + (unsigned)(q % NBUF) * CBUF;
        for (int j = cw; j < NCB; j += CPW) {
            const int b = j < VB0 ? j : SB0 + (j - VB0);
            lds_dma16(src + b * 1024, dst + j * 1024);
        }
    };
    int chain = role.team, c = 0, nch = 0;
    ChainInfo ci{};
    f32x4 S[MT];
    size_t hbase = 0, cbase = 0;   // cbase: h_chunks index of the chain's first chunk
    int hrow = 0;
    bool started = false;
    auto store_hT = [&]() {
        if (computes && args.h_T && hrow >= 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<f32x4 *>(args.h_T + hbase + tile_chan<BF16>(mt, lq, 0)) = S[mt];
        }
    };
    auto open_chain = [&]() {
        ci = chain_info(args, chain);
        nch = (ci.len + CH - 1) / CH;
        c = 0;
        // state row of this sequence: its index, or (pool-addressed) its slot; a
        // negative slot starts from zero and keeps no final state
        hrow = args.state_idx ? args.state_idx[ci.seq] : ci.seq;
        hbase = (((size_t)(hrow < 0 ? 0 : hrow) * args.H + ci.head) * DV + v0 + ln) * DK;
        if (SNAP && computes) {
            // chunks of the sequences before this one
            if (args.cu_seqlens) {
                cbase = 0;
                for (int s2 = 0; s2 < ci.seq; ++s2)
                    cbase += (size_t)((args.cu_seqlens[s2 + 1] - args.cu_seqlens[s2] + CH - 1) / CH);
            } else {
                cbase = (size_t)ci.seq * ((args.T + CH - 1) / CH);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (args.h0 && computes && hrow >= 0)
                S[mt] = *reinterpret_cast<const f32x4 *>(args.h0 + hbase + tile_chan<BF16>(mt, lq, 0));
            else S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        vm_wait<0>();   // the state is never a pending load inside the chunk loop
    };

    // This compute wave's share of chunk q from its LDS buffer; it stores its
    // output tile itself (the compute waves otherwise wait at the step's barrier
    // for the helpers' copies, so the store costs them nothing: measured 2-3 %
    // faster than handing the tile to a helper through LDS).
    auto compute_chunk = [&](int q) {
            const unsigned char *pl = lds + (q % NBUF) * CBUF;
            // v fragment vt of the payload sits in the copied slab blocks, which start at P::V
            const int voff = P::V + P::V + vt * FB - SB0 * 1024;
            // all of this chunk's LDS operands first: their latency overlaps R1
            using FragK = typename std::conditional<BF16, bf16x8, f32x4>::type;
            constexpr int NF = P::NF;
            FragK ak[NF], aq[NF];
            f32x4 eg[MT];
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                ak[s] = *reinterpret_cast<const FragK *>(pl + P::KD + (s * 64 + lane) * 16);
                aq[s] = *reinterpret_cast<const FragK *>(pl + P::QD + (s * 64 + lane) * 16);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) eg[mt] = *reinterpret_cast<const f32x4 *>(pl + P::EG + (16 * mt + 4 * lq) * 4);
            const f32x4 beta = *reinterpret_cast<const f32x4 *>(pl + P::BETA + lq * 16);
            f32x4 vv;
            if constexpr (BF16) {
                const bf16x4 v4 = *reinterpret_cast<const bf16x4 *>(pl + voff + lane * 8);
#pragma unroll
                for (int i = 0; i < 4; ++i) vv[i] = static_cast<float>(v4[i]);
            } else {
                vv = *reinterpret_cast<const f32x4 *>(pl + voff + lane * 16);
            }
            // the state entering this chunk, for the materialised form (same
            // addressing as h_T, chunk row cbase + c); non-temporal stores, so
            // that the snapshots do not evict the payload ring from L2
            if constexpr (SNAP) {
                const size_t at = (((cbase + c) * args.H + ci.head) * DV + v0 + ln) * DK;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    __builtin_nontemporal_store(S[mt], reinterpret_cast<f32x4 *>(args.h_chunks + at + tile_chan<BF16>(mt, lq, 0)));
            }
            // R1: W = k~ S, Qs = q~ S ; then decay the state in place
            f32x4 W = {0.f, 0.f, 0.f, 0.f}, Qs = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BF16) {
#pragma unroll
                for (int s = 0; s < NF; ++s) {
                    bf16x8 b;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        b[i] = static_cast<__bf16>(S[2 * s][i]);
                        b[4 + i] = static_cast<__bf16>(S[2 * s + 1][i]);
                    }
                    W = mfma_bf16(ak[s], b, W);
                    Qs = mfma_bf16(aq[s], b, Qs);
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        W = mfma_f32(ak[mt][i], S[mt][i], W);
                        Qs = mfma_f32(aq[mt][i], S[mt][i], Qs);
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S[mt][i] *= eg[mt][i];
            }
            // R2: u = beta (v - W)
            f32x4 u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = beta[i] * (vv[i] - W[i]);
            // R3: U = INV u ; R4: O = Qs + Mqk U ; R5: S += k^r^T U
            f32x4 U = {0.f, 0.f, 0.f, 0.f}, O;
            if constexpr (BF16) {
                // INV, Mqk and k^r are single bf16 operands, duplicated over both K
                // halves; u and U ride as [hi | lo], so each product is one MFMA
                // with the state-side operand at ~2^-16 relative.
                const bf16x4 inv = *reinterpret_cast<const bf16x4 *>(pl + P::INV + lane * 8);
                const bf16x4 mqk = *reinterpret_cast<const bf16x4 *>(pl + P::MQK + lane * 8);
                bf16x4 uh, ul;
                hilo4(u, uh, ul);
                U = mfma_bf16(dup4(inv), cat4(uh, ul), U);
                bf16x4 Uh, Ul;
                hilo4(U, Uh, Ul);
                const bf16x8 bU = cat4(Uh, Ul);
                O = mfma_bf16(dup4(mqk), bU, Qs);
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
            f32x4 Op;
#pragma unroll
            for (int i = 0; i < 4; ++i) Op[i] = args.scale * O[i];
            // after the quad transpose lane 4c + j holds row 4lq + j, columns 4c .. 4c+3:
            // one 8-byte (bf16) or 16-byte (fp32) store per lane
            const f32x4 b = quad_transpose(Op, ln & 3);
            const int row = 4 * lq + (ln & 3);
            if (row < min(CH, ci.len - c * CH)) {
                const size_t at = ((ci.bos + (size_t)c * CH + row) * args.H + ci.head) * DV + v0 + 4 * (ln >> 2);
                if constexpr (BF16) {
                    uint2 v2;
                    v2.x = pack_bf16x2(b[0], b[1]);
                    v2.y = pack_bf16x2(b[2], b[3]);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(args.o) + at) = v2;
                } else {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(args.o) + at) = b;
                }
            }
    };

    auto next_chunk = [&]() {   // chain bookkeeping (zero-length chains: h_T = h0)
        while (!started || c >= nch) {
            if (started) { store_hT(); chain += args.n_teams; }
            started = true;
            open_chain();
            if (nch == 0) c = 1;
        }
    };

    // Two chunks per step (one barrier per two chunks).  At the top of step st
    // the helpers check chunks 2st+2, 2st+3 ready (from the poll of the previous
    // step), poll and copy payloads 2st+2, 2st+3 into the buffers of the
    // previous step's chunks; they wait for the copies before the barrier,
    // while the compute waves work through chunks 2st, 2st+1.
    auto step2 = [&](int st) {
        const int q0 = 2 * st;
        if (copier) {
            const int spot = st >= 1 ? ((st - 1) & 1) : -1;
            for (int e = 0; e < 2; ++e)
                if (q0 + 2 + e < q_total) ensure_ready(q0 + 2 + e, spot);
            if (cw == 0 && q0 + 4 < q_total) poll_issue(st & 1);
            for (int e = 0; e < 2; ++e)
                if (q0 + 2 + e < q_total) dma(q0 + 2 + e);
            vm_wait<0>();                 // both copies and the poll have landed
        }
        for (int e = 0; e < 2; ++e) {
            if (q0 + e >= q_total) continue;
            next_chunk();
            if (computes) compute_chunk(q0 + e);
            ++c;
        }
        lds_barrier();                    // payloads 2st+2, 2st+3 published; buffers of 2st, 2st+1 free
        if (tid == 64 * NCW) {
            for (int e = 0; e < 2; ++e)
                if (q0 + 2 + e < q_total) add_flag(&used[(q0 + 2 + e) % KDA_RING], 1);
        }
    };

    if (q_total > 0) {
        if (copier) {
            for (int j = 0; j < 2 && j < q_total; ++j) {
                ensure_ready(j, -1);
                dma(j);
            }
            vm_wait<0>();
        }
        lds_barrier();
        if (tid == 64 * NCW) {
            for (int j = 0; j < 2 && j < q_total; ++j) add_flag(&used[j], 1);
        }
    }
    const int nsteps = (q_total + 1) / 2;
    for (int st = 0; st < nsteps; ++st) step2(st);
    // final state of the last open chain, then any trailing zero-length chains
    if (started) store_hT();
    for (chain = started ? chain + args.n_teams : role.team; chain < n_chains; chain += args.n_teams) {
        open_chain();
        store_hT();
    }
}

__global__ __launch_bounds__(256) void chunk_flags_clear_kernel(int *flags, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) flags[i] = 0;
}

template <bool BF16, int DK, int DV, int BDV, bool SNAP>
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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, chunk_fwd_kernel<BF16, DK, DV, BDV, SNAP>, NTHR, 0);
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
    teams_per_xcd = (n_teams + 7) / 8;
    a.teams_per_xcd = teams_per_xcd;
    // paired placement needs two resident workgroups per CU and XCDs of n_cu / 8 CUs
    const int cus_per_xcd = n_cu / 8;
    const int cpt = (TS + 1) / 2;
    a.pair_half = (occ >= 2 && n_cu % 8 == 0 && teams_per_xcd * cpt <= cus_per_xcd) ? cus_per_xcd : 0;
    // flags and the error word start at zero: a small fill kernel (not a memset,
    // so that a caller may capture the launch in a graph)
    hipLaunchKernelGGL(chunk_flags_clear_kernel, dim3(16), dim3(256), 0, stream, a.flags,
                       (int)(chunk_flag_bytes() / sizeof(int)));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned per_xcd = a.pair_half > 0 ? (unsigned)(cus_per_xcd + teams_per_xcd * cpt)
                                             : (unsigned)(teams_per_xcd * TS);
    const unsigned grid = 8u * per_xcd;
    hipLaunchKernelGGL((chunk_fwd_kernel<BF16, DK, DV, BDV, SNAP>), dim3(grid), dim3(NTHR), 0, stream, a);
    return hipGetLastError();
}

// d_v slab width: 32 columns (two compute waves and two helper waves per
// consumer), whatever the number of chains.  Measured on MI355X against 64-
// and 16-column slabs: 1,024 packed chains 5.61 ms (64) -> 4.43 ms (32); 32
// chains of 131,072 tokens 8.14 ms (16) -> 7.49 ms (32); 2..64 chains equal or
// better at 32.
hipError_t launch_chunk_fwd(const ChunkArgs &a, int dtype, int dk, int dv, hipStream_t stream)
{
#define KDA_DISPATCH_S(BF, DKV, DVV, SN) return launch_one<BF, DKV, DVV, 32, SN>(a, stream);
#define KDA_DISPATCH(BF, DKV, DVV)                                             \
    if (dk == DKV && dv == DVV) {                                              \
        if (a.h_chunks) KDA_DISPATCH_S(BF, DKV, DVV, true)                     \
        KDA_DISPATCH_S(BF, DKV, DVV, false)                                    \
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
#undef KDA_DISPATCH_S
    return hipErrorInvalidValue;
}

}  // namespace kda
