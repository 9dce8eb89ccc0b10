// la_walk.h -- one workgroup walking the 64-token chunks of a range of one
// sequence: the chunk pipeline and per-chunk arithmetic shared by the chunk
// kernels.
//
// Per chunk c with tokens i, j = 0..cl-1 (cl = 64 except for a ragged tail),
// decay lambda and S the state before the chunk:
//
//   P[i][j]   = lambda^(i-j) (q_i . k_j)  for j <= i, else 0     (intra scores)
//   o_i       = lambda^(i+1) q_i^T S  +  sum_j P[i][j] v_j          (output)
//   S        <- lambda^cl S + sum_j k_j (lambda^(cl-1-j) v_j)^T     (state)
//
// which is the token recurrence S_t = lambda S_{t-1} + k_t v_t^T,
// o_t = q_t^T S_t regrouped: exact attention inside a chunk and the state
// between chunks (the Lightning Attention-2 split named in the LASP-2 page's
// related-paper list), with the state evaluated right-product-first (LASP-2
// abstract).  Only non-negative powers of lambda are formed, so nothing
// overflows however long the sequence.
//
// Work split inside the workgroup (wave w of NW = D/16):
//   * intra scores: the 10 non-zero 16x16 tiles of P^T = K Q^T are dealt
//     round-robin to the waves and written to LDS as P[i][j];
//   * wave w owns state columns v in [16 w, 16 w + 16): its slice of S stays
//     in registers, serves directly (rounded to bf16) as the A operand of
//     O^T = S^T Q^T, and is updated by S += K^T (diag(lambda^(cl-1-j)) V);
//   * outputs are produced as O^T tiles so each lane ends up with 4
//     consecutive v of one token: one 8-byte (bf16) store per tile.
//
// Memory pipeline: Q, K, V chunks go from HBM straight into LDS (16 bytes
// per lane, no register staging) through STAGES buffers, so STAGES-1 chunks
// are in flight while one is computed.  LDS holds only token-major tiles
// (rows padded to an odd number of 16-byte granules; each lane's 16 B of a
// load land where its row and piece put them) plus P; operands that contract
// over tokens (K^T, V^T) use the gfx950 transposing LDS read, so no
// transposed copy is ever written.  Token and feature orders inside the MFMA
// steps are chosen so that no LDS access has a bank conflict.  A
// ragged tail loads clamped (valid, finite) rows past the end and masks them
// out through the decay factors.  Two barriers per chunk, without fences:
// waits are explicit.
#pragma once

#include "la_device.h"

namespace la {


// The 10 lower-triangular (key block jb <= query block ib) tiles of the
// 64x64 score matrix, dealt round-robin to the waves.
__device__ inline void score_tile(int idx, int& jb, int& ib) {
  if (idx < 4) { jb = idx; ib = idx; }
  else if (idx < 7) { jb = idx - 4; ib = idx - 3; }
  else if (idx < 9) { jb = idx - 7; ib = idx - 5; }
  else { jb = 0; ib = 3; }
}

constexpr int LDS_MAX = 160 * 1024;  // per workgroup on gfx950


// Position of token t (0..63) in a gated walk's per-chunk factor tables
// (cumulative log-gate c_t, update weight exp(c_last - c_t)), chosen so that
// the values a lane needs sit together: the 16 update-weight slots of MFMA
// lane group g (tokens slot_token) are entries 16 g .. 16 g + 15 in slot
// order, and the 4 keys of group g in key block jb (score tile rows) are
// entries 16 g + 4 jb .. + 3.
template <typename T>
__device__ inline int tab_pos(int t) {
  if constexpr (sizeof(T) == 2) {
    // group of t: t mod 8 in {0, 2} -> 0, {4, 6} -> 1, {5, 7} -> 2, {1, 3} -> 3
    // (the token sets tr_row gives lane groups 0..3); slot order inside
    const int grp = (0x2130 >> (4 * (((t >> 2) & 1) * 2 + (t & 1)))) & 3;
    return 16 * grp + 2 * (t >> 3) + ((t >> 1) & 1);
  } else {
    return 16 * (t & 3) + (t >> 2);  // group g = t mod 4, slot js = t / 4
  }
}

// LDS of a workgroup: STAGES stages of NSLOT token-major tiles (Q, K, V when
// NSLOT = 3, K, V when NSLOT = 2, the four tensors of NH = 2 walks that share
// their keys and values crosswise when NSLOT = 4, or of one walk that also
// accumulates a second state (Q, K, V, Q2) when NSLOT = 4 and NH = 1), plus
// one P per walk when NSLOT >= 3, plus (gated walks)
// a ring of STAGES + 1 slots of 64 log-gates (a chunk's gates travel with
// the previous chunk's tiles, one chunk ahead of them) and two buffers of the
// chunk factor tables (GateTab).
template <typename T, int D, int NSLOT, bool GATED = false, int NH = 1>
struct FwdLayout {
  typedef PadTile<T, CH, D> TN;                // Q, K, V token-major [token][d]
  typedef PBlocks<T> TP;                       // P, its 10 nonzero 16x16 blocks
  static_assert(NH == 1 || NSLOT == 4, "two walks share a stage of four tiles");
  static constexpr int NTEN = NSLOT;           // tensor tiles per stage
  static constexpr int TB = TN::BYTES;         // one tensor tile
  static constexpr int STAGE = NTEN * TB;
  static constexpr int PBYTES = NSLOT >= 3 ? NH * TP::BYTES : 0;  // one P per walk
  static constexpr int SMAX = NSLOT >= 3 ? 3 : 5;
  static constexpr int GB = GATED ? CH * 4 : 0;  // log-gates of one chunk
  static constexpr int TBL = GATED ? 2 * 2 * CH * 4 : 0;  // 2 x (cumulative gate, update weight)
  static constexpr int NW = D / 16;  // waves: one per 16 state columns
  static constexpr int UB = (NSLOT == 4 && NH == 1) ? CH * 4 : 0;
  static constexpr int SFIT = (LDS_MAX - PBYTES - GB - TBL - UB) / (STAGE + GB);
  static constexpr int STAGES = SFIT < SMAX ? SFIT : SMAX;
  static constexpr int OFF_P = STAGES * STAGE;
  static constexpr int OFF_G = OFF_P + PBYTES;
  static constexpr int GSLOTS = STAGES + 1;  // gate ring (gated walks)
  static constexpr int OFF_T = OFF_G + GSLOTS * GB;
  static constexpr int OFF_U = OFF_T + TBL;  // (one walk of four tiles) weights of its second state
  static constexpr int BYTES = OFF_U + UB;
  static constexpr int NT = 64 * NW;
  // bf16 keeps two waves per SIMD (256 registers per lane)
  static constexpr int WAVES_PER_EU = sizeof(T) == 2 ? 2 : 1;
  static_assert(STAGES >= 1 && STAGES <= 5 && BYTES <= LDS_MAX, "LDS budget");
  static_assert(TB == TN::G * 1024, "a tile is G loads of 1 KiB");
};

// wait until chunk c's loads have landed (loads of `later` younger chunks,
// LPC per chunk, may still be in flight), then barrier
template <int LPC, int MAXLATER>
__device__ inline void wait_chunk_n(int later) {
  if constexpr (MAXLATER >= 3) {
    if (later >= 3) { wait_vm_barrier<3 * LPC>(); return; }
  }
  if constexpr (MAXLATER >= 2) {
    if (later >= 2) { wait_vm_barrier<2 * LPC>(); return; }
  }
  if constexpr (MAXLATER >= 1) {
    if (later >= 1) { wait_vm_barrier<LPC>(); return; }
  }
  wait_vm_barrier<0>();
}
// the same for a wave in load-count class cls (0, 1, 2: L0, L1 or L2 loads
// per chunk)
template <int L0, int L1, int L2, int MAXLATER>
__device__ inline void wait_chunk3(int cls, int later) {
  if (cls == 0)
    wait_chunk_n<L0, MAXLATER>(later);
  else if (cls == 1)
    wait_chunk_n<L1, MAXLATER>(later);
  else
    wait_chunk_n<L2, MAXLATER>(later);
}


// A range of one sequence for walk(): positions t0 .. t0+len-1 (position tt
// is row tt, or row Ls-1-tt when reverse), all pointers at the sequence's
// first row.
struct WalkJob {
  const void* Q;  // read only when outputs are formed
  const void* K;
  const void* V;
  void* O;        // written when outputs are formed
  int64_t t0;
  int len;        // positions; fits in int (one sequence spans under 4 GiB)
  int64_t Ls;
  int reverse;
  float lg;       // log2 lambda (fixed-decay walks)
  const float* G; // log-gates of the sequence, [Ls] (gated walks)
  int last_chunk_first;  // state-only walks over whole chunks: chunks in reverse order
  // fixed decay: the start state already carries the first token's decay,
  // so the first chunk decays it by lambda^(i) and lambda^(cl-1) instead of
  // lambda^(i+1) and lambda^cl
  int first_undecayed;
  // NH = 2 walks: the four tensors a stage holds (slots 0..3: the first
  // walk's Q, the second's Q, the first's K, the first's V; the second walk's
  // K and V are the first's V and K).  Set in the first job.
  const void* src4[4];
  // one walk of four tiles (NSLOT = 4, NH = 1): the keys of its second state
  // U = sum_t lambda^(t - t0) Q2_t Q_t^T (its values are this walk's queries)
  const void* Q2;
  // RK, last job (bf16 at d = 128): per position, rk[row] = (this walk's
  // output row) . (the first walk's query row when NH = 2, the Q2 row for
  // one walk of four tiles) over the bf16 outputs, in fp32; sequence base
  // like the tensors
  float* rk;
  // output walks built with DUMP (may be null): after every chunk that ends on a boundary
  // row y = m * 2^dump_shift (0 < y < Ls) of the sequence, this walk's state
  // goes to dump[slot] ([ndump][D][D], the sequence's own), slot m - 1, or
  // ndump - m when dump_rev (numbered from the end)
  float* dump;
  int dump_shift, ndump, dump_rev;
};

// Walk the range with the state in accS (wave w: columns [16 w, 16 w + 16),
// accumulator tile tk holds rows 16 tk + 4 g + r); accS ends as the state
// after the range.  OUT: also form and store the outputs.  NSLOT: tiles per
// LDS stage of the caller's layout (the K, V slots are the last two).  All
// of the workgroup's threads call it; LDS is free again on return.
//
// GATED: the decay is a per-token gate alpha_t = exp(g_t) (the data-dependent
// gates of the Gated Linear Attention entry of the LASP-2 page's
// related-paper list, one scalar per token and head):
//   S_t = alpha_t S_{t-1} + k_t v_t^T.
// With c_i = g_0 + .. + g_i the chunk-local cumulative log-gate, every
// factor above becomes a difference of c: lambda^(i-j) -> exp(c_i - c_j),
// lambda^(i+1) -> exp(c_i), lambda^(cl-1-j) -> exp(c_{cl-1} - c_j),
// lambda^cl -> exp(c_{cl-1}); all are <= 1.  Wave NW-1 brings each chunk's
// 64 gates to LDS together with the previous chunk's tiles, forms c with a
// wave-wide prefix sum (lane = token) and writes c and the update weights
// exp(c_{cl-1} - c_j) to a table (tab_pos order) while chunk c - 1's update
// runs; after the next barrier every wave reads the factors it needs with a
// few vector LDS reads instead of gathering them lane by lane.  Returns the
// range's total log-gate (0 if not GATED).
//
// NH = 2: every wave walks two recurrences side by side over the same
// positions with the same decay (jbs[0], jbs[1]; state h in accS[h]) whose
// keys and values are crosswise the same tensors: the backward's dV and dK
// sweeps, both over q dO^T (keys Q, values dO, queried by K; keys dO, values
// Q, queried by V).  A stage then holds four tiles instead of six, the two
// share every load, barrier and decay factor, and each wave has two
// independent streams of matrix products to interleave.
//
// NSLOT = 4 with NH = 1 (fixed decay, outputs): the walk also accumulates
// U = sum_t lambda^(t - t0) q2_t q_t^T over its positions from zero into
// accU (same column split as the state; keys Q2 = jb.Q2, values this walk's
// queries), the weights growing with the position instead of decaying a
// state.  The backward's dQ sweep (queries dO) takes Q2 = Q: U is then the
// local state of each sub-segment for the reverse dV and dK sweeps, formed
// from the dO tiles the dQ sweep reads anyway instead of by a pre-pass that
// reads Q and dO again.
template <typename T, int D, bool OUT, int NSLOT, bool GATED = false, int NH = 1, bool RK = false,
          bool DUMP = false>
__device__ __forceinline__ float walk(char* smem, const WalkJob (&jbs)[NH],
                                      f32x4 (&accS)[NH][D / 16], f32x4* accU = nullptr) {
  typedef Elt<T> X;
  typedef typename X::op_t op_t;
  typedef FwdLayout<T, D, NSLOT, GATED, NH> LY;
  constexpr bool ACCU = NSLOT == 4 && NH == 1;
  static_assert(NSLOT >= 3 || !OUT, "outputs need the Q slot and P");
  static_assert(NH == 1 || (OUT && NSLOT == 4), "two walks form outputs from four tiles");
  static_assert(!ACCU || OUT, "the second state rides on an output walk");
  const WalkJob& jb = jbs[0];  // positions, direction, decay: shared
  typedef typename LY::TN TN;
  typedef typename LY::TP TP;
  constexpr int E = X::E;           // operand elements per lane
  constexpr int KS = 4 * E;         // MFMA contraction step
  constexpr int NW = LY::NW;        // waves
  constexpr int EP = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int NKT = D / 16;       // 16-high state-row tiles
  constexpr int NST = (10 + NW - 1) / NW;  // score tiles per wave (at most)
  constexpr int NKS = D / KS;       // contraction steps over d
  constexpr int NJS = CH / KS;      // contraction steps over a chunk
  constexpr int S = LY::STAGES;
  constexpr int TB = LY::TB;
  constexpr int G = TN::G;
  // one chunk is NLOAD * G loads of 1 KiB (64 lanes x 16 B) into slots
  // SLOT0.. (see the chunk loads below)
  constexpr int NLOAD = (NH == 2 || ACCU) ? 4 : (OUT ? 3 : 2);
  constexpr int SLOT0 = NSLOT - NLOAD;
  // stage slots of walk h's Q, K, V tiles
  auto qslot = [](int h) { return NH == 2 ? h : 0; };
  auto kslot = [](int h) { return NH == 2 ? 2 + h : (NSLOT >= 3 ? 1 : 0); };
  auto vslot = [](int h) { return NH == 2 ? 3 - h : (NSLOT >= 3 ? 2 : 1); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int col = 16 * w;  // this wave's state columns [col, col + 16)

  const float lg = jb.lg;
  const int64_t t0 = jb.t0;
  const int len = jb.len;
  const int nch = (len + CH - 1) / CH;

  // Rows of sequence n are addressed relative to its first row (byte offsets
  // within one sequence fit in 32 bits; the host checks that).  relrow(tt)
  // is the row of position tt of this sub-segment; consecutive chunks are
  // `dir * CH` rows apart.
  auto relrow = [&](int64_t tt) -> int64_t { return jb.reverse ? (jb.Ls - 1 - (t0 + tt)) : (t0 + tt); };
  const int cstride_b = (jb.reverse ? -1 : 1) * CH * D * (int)sizeof(T);  // bytes per chunk
  // last chunk first (state-only walks over whole chunks): step c takes chunk
  // nch-1-c, and its update weights carry the decay of the c chunks after it
  // (lambda^(cl-1-j + CH c); gated: exp(c_last - c_j) times the gates of the
  // chunks already walked) instead of decaying the state
  const bool lcf = !OUT && jb.last_chunk_first && len % CH == 0;
  auto phys = [&](int c) { return lcf ? nch - 1 - c : c; };

  // ---- chunk loads: HBM -> LDS, 1 KiB (64 lanes x 16 B) per instruction.
  // Block blk (0..G-1) of a tile is granules 64 blk .. + 63; lane l's granule
  // is (row, piece) = divmod(64 blk + l, G), the last piece of a row being
  // padding (it loads the row's first piece).  Wave w takes blocks w, w + NW,
  // ... and loads each of them for all NLOAD tiles, whose offsets within a
  // tile agree: NBW offsets per lane, those of chunk 0 precomputed; a ragged
  // last chunk clamps rows past the end to the last valid token.
  // Per chunk a wave issues nbw * NLOAD tile loads (nbw = NBW or NBW - 1),
  // wave NW-1 one more for the gates: chunk c's group carries the gates of
  // chunk c + 1 (of the last chunk again at the end, so the count never
  // changes); chunk 0's gates are one extra load issued before any tile,
  // older than everything the waits count.
  constexpr int NBW = (G + NW - 1) / NW;  // blocks of the busiest wave
  static_assert(G > NW, "every wave loads at least one block");
  constexpr int NBW_LAST = (G - (NW - 1) + NW - 1) / NW;  // blocks of wave NW-1
  const int nbw = (G - w + NW - 1) / NW;                  // this wave's (wave-uniform)
  const bool gwave = GATED && (w == NW - 1);
  // per-wave load count class for the waits: NBW blocks, NBW - 1, or the
  // gate wave's blocks plus its gate load
  const int wcls = gwave ? 2 : (nbw == NBW ? 0 : 1);
  auto tensor_base = [&](int ten) -> const T* {
    // (selects, not an indexed array: the base must stay wave-uniform)
    const void* bp =
        NH == 2 ? (ten == 0 ? jb.src4[0] : ten == 1 ? jb.src4[1] : ten == 2 ? jb.src4[2] : jb.src4[3])
        : ACCU  ? (ten == 0 ? jb.Q : ten == 1 ? jb.K : ten == 2 ? jb.V : jb.Q2)
        : OUT   ? (ten == 0 ? jb.Q : (ten == 1 ? jb.K : jb.V))
                : (ten == 0 ? jb.K : jb.V);
    return reinterpret_cast<const T*>(bp);
  };
  auto piece_off = [&](int blk, int& row) -> int {  // lane's row and piece offset (elements)
    const int pos = 64 * blk + lane;
    row = pos / G;
    const int pc = pos % G;
    return ((pc == G - 1) ? 0 : pc) * EP;
  };
  unsigned voff0[NBW];  // chunk-0 byte offset of this lane's piece, per block
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    const int blk = (w + NW * k < G) ? w + NW * k : 0;
    int row;
    const int po = piece_off(blk, row);
    voff0[k] = (unsigned)((relrow(row) * D + po) * (int64_t)sizeof(T));
  }
  const unsigned smem_lds = lds_address(smem);
  // gates of chunk cg into the gate slot of chunk number `slot_of`
  auto gate_slot = [&](int cc) -> int { return cc % LY::GSLOTS; };
  auto issue_gates = [&](int cg, int slot_of) {
    const int pg = phys(cg);
    const int tt = (pg * CH + lane < len) ? pg * CH + lane : len - 1;
    dma4(jb.G, (unsigned)(relrow(tt) * 4),
         smem_lds + (unsigned)(LY::OFF_G + gate_slot(slot_of) * LY::GB));
  };
  // chunk c into stage `stage`; offsets wrap modulo 2^32 like the byte
  // offsets they stand for (the host keeps one sequence below 4 GiB)
  auto issue = [&](int cs, int stage) {
    const unsigned sb = smem_lds + (unsigned)(stage * LY::STAGE);
    const int c = phys(cs);
    const bool full = (c + 1) * CH <= len;
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
      if (k < NBW - 1 || nbw == NBW) {
        const int blk = w + NW * k;
        unsigned voff;
        if (full) {
          voff = voff0[k] + (unsigned)c * (unsigned)cstride_b;
        } else {
          int row;
          const int po = piece_off(blk, row);
          const int tt = (c * CH + row < len) ? c * CH + row : len - 1;
          voff = (unsigned)((relrow(tt) * D + po) * (int64_t)sizeof(T));
        }
#pragma unroll
        for (int ten = 0; ten < NLOAD; ++ten)
          dma16(tensor_base(ten), voff, sb + (unsigned)((SLOT0 + ten) * TB + blk * 1024));
      }
    }
    if (GATED && gwave) issue_gates(cs + 1 < nch ? cs + 1 : nch - 1, cs + 1);
  };

  // first chunks in flight while the factors are computed
  if (GATED && gwave && nch > 0) issue_gates(0, 0);
  for (int pc = 0; pc < S - 1; ++pc)
    if (pc < nch) issue(pc, pc);

  // ---- factors
  float qf[4];        // lambda^(i+1) for the lane's query i of each 16-row block
  float pf[NST][4];   // lambda^(i-j) (or 0) for the wave's score tiles
  auto set_pf = [&](int cl) {
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int idx = w + NW * st;
      int jb = 0, ib = 0;
      if (idx < 10) score_tile(idx, jb, ib);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // accumulator (row 4 g + r, column l16) of tile (jb, ib) holds P[i][j]
        const int i = 16 * ib + perm16<T>(l16), j = 16 * jb + perm16<T>(4 * g + r);
        pf[st][r] = (idx < 10 && j <= i && j < cl) ? pow_lam(lg, (float)(i - j)) : 0.0f;
      }
    }
  };
  T* Oseq[NH];  // sequence base of each walk's O
#pragma unroll
  for (int h = 0; h < NH; ++h) Oseq[h] = reinterpret_cast<T*>(jbs[h].O);
  // bf16 at d = 128 (8 waves x 16 columns, 256-byte rows): a chunk's outputs
  // are staged in LDS and stored as whole rows with non-temporal stores (the
  // rows are written once and never read here, so they do not displace the
  // K, V lines the state pre-pass left in the last-level cache); storing each
  // lane's 8-byte piece directly sends every 128-byte line to L2 in four
  // pieces from four waves.  Measured at 64K tokens x 32 heads: whole call
  // 582.7 -> 564.1 us (plain whole-row stores: no gain).  Not so for two
  // walks without row dots (the backward's joint dV/dK walk): there the
  // staging's two barriers per chunk cost more than the merged lines save,
  // and its outputs go straight out in 8-byte pieces (plain stores; as
  // non-temporal pieces the walk took half as long again).
  constexpr bool OSTAGE = OUT && sizeof(T) == 2 && D == 128 && !(NH == 2 && !RK);
  T ohold[NH][4][4];
  // RK: row dots of the last walk's outputs with the first walk's queries
  // (NH = 2) or with Q2 (one walk of four tiles), per position to the last
  // job's rk
  constexpr bool rkw = RK && (NH == 2 || ACCU) && OSTAGE;
  static_assert(!RK || rkw, "row dots: two walks or four tiles, bf16 at d = 128");
  unsigned ooff0[4];  // element offset (chunk 0) of the lane's outputs in each 16-row block
  const bool und = !GATED && jb.first_undecayed;  // wave-uniform
  // lambda^(i+1) (or lambda^i for a start state that already carries the
  // first token's decay) for the lane's query i of each 16-row block
  auto set_qf = [&](int shift) {
#pragma unroll
    for (int it = 0; it < 4; ++it) qf[it] = pow_lam(lg, (float)(16 * it + l16 + shift));
  };
  if (OUT) {
#pragma unroll
    for (int it = 0; it < 4; ++it) ooff0[it] = (unsigned)(relrow(16 * it + l16) * D + col + 4 * g);
    if (!GATED) {
      set_qf(und ? 0 : 1);
      set_pf(CH);
    }
  }
  const float lamC = GATED ? 0.0f : pow_lam(lg, (float)CH);
  // lambda^(cl-1-j) (0 past the tail) for the lane's contraction slots j of the update
  float wv[NJS][E];
  auto set_wv = [&](int cl) {
#pragma unroll
    for (int js = 0; js < NJS; ++js)
#pragma unroll
      for (int x = 0; x < E; ++x) {
        const int j = slot_token<T>(js * KS, g, x);
        wv[js][x] = (j < cl) ? pow_lam(lg, (float)(cl - 1 - j)) : 0.0f;
      }
  };
  if (!GATED) set_wv(CH);
  // ACCU: lambda^j for the lane's contraction slots j of a chunk, in slot
  // order (entry 16 g + E js + x), visible after the loop's first barrier
  float* const tabU = reinterpret_cast<float*>(smem + LY::OFF_U);
  if constexpr (ACCU) {
    if (tid < 64) {
      const int js = (tid & 15) / E, x = (tid & 15) % E;
      tabU[tid] = pow_lam(lg, (float)slot_token<T>(js * KS, tid >> 4, x));
    }
  }
  float gsum2 = 0.0f;  // total log2-gate of the chunks walked (GATED)
  float gchunk2 = 0.0f;  // (GATED) the current chunk's total log2-gate
  float ug0 = 0.0f;      // (GATED, ACCU) log2-gate of the walk's first token
  float dc = GATED ? 0.0f : lamC;  // decay of the state over the current chunk

  // GATED, wave NW-1: the factor tables of chunk cc (its gates are in LDS
  // and visible) into buffer cc % 2
  float gwalked2 = 0.0f;  // (lcf) total log2-gate of the chunks walked, wave NW-1
  auto write_tables = [&](int cc) {
    const int cl = (len - cc * CH < CH) ? (len - cc * CH) : CH;
    // chunk-local cumulative log-gate in log2 units, lane = token
    const float c2 = wave_prefix_sum(
        *reinterpret_cast<const float*>(smem + LY::OFF_G + gate_slot(cc) * LY::GB + 4 * lane) *
        1.4426950408889634f);
    const float clast = lane_value(c2, cl - 1);
    const float ew = (lane < cl) ? exp2_np(clast - c2 + gwalked2) : 0.0f;  // update weight
    if (lcf) gwalked2 += clast;
    float* tab = reinterpret_cast<float*>(smem + LY::OFF_T + (cc & 1) * 2 * CH * 4);
    const int pos = tab_pos<T>(lane);
    tab[pos] = c2;
    tab[CH + pos] = ew;
  };
  // GATED, every wave: the factors of chunk cc from its tables
  auto read_factors = [&](int cc) {
    const int cl = (len - cc * CH < CH) ? (len - cc * CH) : CH;
    const float* tab = reinterpret_cast<const float*>(smem + LY::OFF_T + (cc & 1) * 2 * CH * 4);
    const float clast = tab[tab_pos<T>(cl - 1)];
    gsum2 += clast;
    gchunk2 = clast;
    dc = lcf ? 1.0f : exp2_np(clast);
    // update weights of the lane's contraction slots
    if constexpr (E == 8) {
#pragma unroll
      for (int js = 0; js < NJS; ++js) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(tab + CH + 16 * g + 8 * js);
        const f32x4 b = *reinterpret_cast<const f32x4*>(tab + CH + 16 * g + 8 * js + 4);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          wv[js][x] = a[x];
          wv[js][4 + x] = b[x];
        }
      }
    } else {
#pragma unroll
      for (int js = 0; js < NJS; js += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(tab + CH + 16 * g + js);
#pragma unroll
        for (int x = 0; x < 4; ++x) wv[js + x][0] = a[x];
      }
    }
    if (OUT) {
#pragma unroll
      for (int it = 0; it < 4; ++it) qf[it] = exp2_np(tab[tab_pos<T>(16 * it + l16)]);
#pragma unroll
      for (int sti = 0; sti < NST; ++sti) {
        const int idx = w + NW * sti;
        int jb_ = 0, ib_ = 0;
        if (idx < 10) score_tile(idx, jb_, ib_);
        const int i = 16 * ib_ + perm16<T>(l16);
        const float ci = tab[tab_pos<T>(i)];
        float cj[4];
        if constexpr (sizeof(T) == 2) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(tab + 16 * g + 4 * jb_);
#pragma unroll
          for (int r = 0; r < 4; ++r) cj[r] = a[r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) cj[r] = tab[tab_pos<T>(16 * jb_ + perm16<T>(4 * g + r))];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jb_ + perm16<T>(4 * g + r);
          pf[sti][r] = (idx < 10 && j <= i && j < cl) ? exp2_np(ci - cj[r]) : 0.0f;
        }
      }
    }
  };

  int st = 0;             // stage holding chunk c
  int st_next = S - 1;    // stage for chunk c + S - 1 (the one chunk c - 1 used)
  for (int c = 0; c < nch; ++c) {
    const int cl = (len - c * CH < CH) ? (len - c * CH) : CH;
    if constexpr (S == 1) {
      lds_barrier();  // the previous chunk's LDS reads are done
      issue(c, 0);
      wait_vm_barrier<0>();
    } else {
      const int later = (nch - 1 - c < S - 2) ? nch - 1 - c : S - 2;
      // chunk c landed; chunk c-1 consumed
      wait_chunk3<NBW * NLOAD, (NBW - 1) * NLOAD, NBW_LAST * NLOAD + 1, S - 2>(wcls, later);
      if (c + S - 1 < nch) issue(c + S - 1, st_next);
      st_next = (st_next + 1 == S) ? 0 : st_next + 1;
    }
    if constexpr (GATED) {
      if (c == 0) {  // later chunks' tables are written one chunk ahead
        if (gwave) write_tables(0);
        lds_barrier();
      }
      // the next chunk's tables, now: its gates came with this chunk's tiles,
      // its buffer was last read in the previous chunk, and the gate wave
      // (one score tile fewer than the busiest waves) has time for them
      // before the scores' barrier, where at the chunk's end every wave
      // waited for it at the next barrier
      if (gwave && c + 1 < nch) write_tables(c + 1);
      read_factors(c);
    } else {
      if (cl != CH) {
        set_wv(cl);
        if (OUT) set_pf(cl);
      }
      dc = lcf ? 1.0f : ((cl == CH) ? lamC : pow_lam(lg, (float)cl));
      if (und) {
        if (c == 0) dc = pow_lam(lg, (float)(cl - 1));
        if (OUT && c == 1) set_qf(1);
      }
    }
    const char* const stage = smem + st * LY::STAGE;
    st = (st + 1 == S) ? 0 : st + 1;

    // V^T operands of this wave's columns (intra A operand; scaled: update B operand)
    op_t Vop[NH][NJS];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int js = 0; js < NJS; ++js)
        Vop[h][js] = tr_op<T, TN>(stage + vslot(h) * TB, js * KS, col, lane);

    // ---- ACCU: U += Q2^T (diag(w_j) Q), 0 past the tail (before the outputs
    // are staged in the Q tile); w_j = lambda^(64 c + j), gated the product of
    // the gates of the walk's tokens after its first up to token j:
    // exp2(c_j + log2-gates of the earlier chunks - log2-gate of the first)
    if constexpr (ACCU) {
      const char* const sQ = stage + qslot(0) * TB;
      const char* const sU = stage + 3 * TB;
      float wu[NJS][E];
      if constexpr (GATED) {
        const float* tab = reinterpret_cast<const float*>(smem + LY::OFF_T + (c & 1) * 2 * CH * 4);
        if (c == 0) ug0 = tab[tab_pos<T>(0)];
        const float gb = gsum2 - gchunk2 - ug0;
#pragma unroll
        for (int js = 0; js < NJS; ++js)
#pragma unroll
          for (int x = 0; x < E; ++x) {
            const float e = exp2_np(gb + tab[16 * g + E * js + x]);  // slot order
            wu[js][x] = (cl == CH || slot_token<T>(js * KS, g, x) < cl) ? e : 0.0f;
          }
      } else if (cl == CH) {
        const float fu = pow_lam(lg, (float)(CH * c));  // lambda^(64 c)
#pragma unroll
        for (int js = 0; js < NJS; ++js)
#pragma unroll
          for (int x = 0; x < E; ++x) wu[js][x] = tabU[16 * g + E * js + x] * fu;
      } else {
#pragma unroll
        for (int js = 0; js < NJS; ++js)
#pragma unroll
          for (int x = 0; x < E; ++x) {
            const int j = slot_token<T>(js * KS, g, x);
            wu[js][x] = j < cl ? pow_lam(lg, (float)(CH * c + j)) : 0.0f;
          }
      }
      op_t Bu[NJS];
#pragma unroll
      for (int js = 0; js < NJS; ++js) {
        const op_t Qop = tr_op<T, TN>(sQ, js * KS, col, lane);
        if constexpr (E == 8) {
          bf16x8 b;
#pragma unroll
          for (int x = 0; x < 8; ++x) b[x] = (__bf16)((float)Qop[x] * wu[js][x]);
          Bu[js] = b;
        } else {
          Bu[js] = Qop * wu[js][0];
        }
      }
#pragma unroll
      for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          const op_t Au = tr_op<T, TN>(sU, js * KS, 16 * tk, lane);
          accU[tk] = X::mfma(Au, Bu[js], accU[tk]);
        }
    }
    if (OUT) {
      // ---- intra scores: P^T tiles = K Q^T, masked and decayed, to LDS as P[i][j]
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const char* const sQ = stage + qslot(h) * TB;
        const char* const sK = stage + kslot(h) * TB;
        char* const sP = smem + LY::OFF_P + h * TP::BYTES;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int idx = w + NW * st;
          if (idx < 10) {
            int jb, ib;
            score_tile(idx, jb, ib);
            // operand row l16 is token perm16(l16) of the block; the
            // contraction over d visits features in score_granule order
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int rk = 16 * jb + perm16<T>(l16), rq = 16 * ib + perm16<T>(l16);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
              const int f = (E == 8) ? 8 * score_granule<D>(ks, g) : ks * KS + g;
              const op_t A = lds_op<T>(sK, TN::off(rk, f));
              const op_t B = lds_op<T>(sQ, TN::off(rq, f));
              acc = X::mfma(A, B, acc);
            }
            T pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[r] = X::from_f(acc[r] * pf[st][r]);
            // keys perm16(4 g + r), r = 0..3, form slab g; query row perm16(l16)
            char* dst = sP + TP::at(ib, jb, g, perm16<T>(l16));
            if (sizeof(T) == 2)
              *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<u32x2*>(pv);
            else
              *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(pv);
          }
        }
      }
      lds_barrier();  // P complete

#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const char* const sQ = stage + qslot(h) * TB;
        const char* const sP = smem + LY::OFF_P + h * TP::BYTES;
        // ---- state before this chunk as the A operand of O^T = S^T Q^T
        op_t Sop[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if constexpr (E == 8) {
            bf16x8 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              o[r] = (__bf16)accS[h][2 * ks][r];
              o[4 + r] = (__bf16)accS[h][2 * ks + 1][r];
            }
            Sop[ks] = o;
          } else {
            Sop[ks] = accS[h][ks / 4][ks % 4];
          }
        }

        // ---- outputs, one 16-token block at a time
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int i = 16 * it + l16;
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
          // inter: sum_k S[k][v] q_i[k], with Q read in the permuted slot order
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            op_t B;
            if constexpr (E == 8) {
              const u32x2 lo = lds_read8(sQ + TN::off(i, 32 * ks + 4 * g));
              const u32x2 hi = lds_read8(sQ + TN::off(i, 32 * ks + 16 + 4 * g));
              const u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
              B = __builtin_bit_cast(bf16x8, both);
            } else {
              B = *reinterpret_cast<const float*>(sQ + TN::off(i, 16 * (ks / 4) + 4 * g + (ks % 4)));
            }
            o = X::mfma(Sop[ks], B, o);
          }
          o *= qf[it];
          // intra: sum_j V^T[v][j] P[i][j] over key blocks jb <= it; slab g of
          // a block holds exactly the keys of lane group g's slots
#pragma unroll
          for (int js = 0; js < NJS; ++js) {
            if (js * KS < 16 * (it + 1)) {
              op_t Bp;
              if constexpr (E == 8) {
                const u32x2 z = {0u, 0u};
                const u32x2 lo = lds_read8(sP + TP::at(it, 2 * js, g, l16));
                const u32x2 hi =
                    (2 * js + 1 <= it) ? lds_read8(sP + TP::at(it, 2 * js + 1, g, l16)) : z;
                const u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
                Bp = __builtin_bit_cast(bf16x8, both);
              } else {
                const int j = js * KS + g;
                Bp = ((j >> 4) <= it)
                         ? *reinterpret_cast<const float*>(
                               sP + TP::at(it, j >> 4, (j & 15) >> 2, l16) + (j & 3) * (int)sizeof(T))
                         : 0.0f;
              }
              o = X::mfma(Vop[h][js], Bp, o);
            }
          }
          // store: lane holds O[token i][v0 .. v0+3]
          if constexpr (OSTAGE) {
            // held until every wave is done with the chunk's Q tile
#pragma unroll
            for (int r = 0; r < 4; ++r) ohold[h][it][r] = X::from_f(o[r]);
          } else if (c * CH + i < len) {
            T* orow = Oseq[h] + (ooff0[it] + (unsigned)c * (unsigned)(cstride_b / (int)sizeof(T)));
            T ov[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ov[r] = X::from_f(o[r]);
            if (sizeof(T) == 2)
              // (bf16 at d = 64: 32-byte pieces of 16 rows, merged in L2)
              *reinterpret_cast<u32x2*>(orow) = *reinterpret_cast<u32x2*>(ov);
            else
              *reinterpret_cast<u32x4*>(orow) = *reinterpret_cast<u32x4*>(ov);
          }
        }
      }
    }

    // ---- the chunk's O tile through LDS: each wave writes its 16 columns of
    // every token, then stores 8 whole rows, 16 bytes per lane.  One walk:
    // through its V tile, right after the outputs (one barrier: nothing reads
    // that tile after the chunk's V operands).  Two walks (NH = 2): after
    // the state updates, through the tiles no longer read then (the first
    // walk's keys, the second walk's queries), so that the first walk's
    // queries stay in place; RK dots them with the second walk's output rows
    // on the way out.
    auto flush_o = [&]() {
      // one walk: its V tile, read only into registers at the chunk's start
      // (so every wave is done with it since the scores' barrier)
      auto oslot = [&](int h) { return NH == 2 ? (h == 0 ? 2 : 1) : vslot(0); };
      if constexpr (NH == 2) lds_barrier();  // every wave is done reading the tiles written below
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        char* const sO = const_cast<char*>(stage + oslot(h) * TB);
#pragma unroll
        for (int it = 0; it < 4; ++it)
          *reinterpret_cast<u32x2*>(sO + TN::off(16 * it + l16, col + 4 * g)) =
              *reinterpret_cast<const u32x2*>(ohold[h][it]);
      }
      lds_barrier();
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const char* const sO = stage + oslot(h) * TB;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = 8 * w + 4 * hh + (lane >> 4);  // 16 lanes per 256-byte row
          const int piece = lane & 15;
          const bool valid = c * CH + row < len;
          if (rkw && h == NH - 1) {
            const u32x4 val = *reinterpret_cast<const u32x4*>(sO + TN::off(row, 8 * piece));
            const int dslot = NH == 2 ? qslot(0) : 3;  // the rows dotted with
            const u32x4 kq =
                *reinterpret_cast<const u32x4*>(stage + dslot * TB + TN::off(row, 8 * piece));
            // (bf16 only: two products a step into the fp32 sum, no conversions;
            // the pairs are copied out of the vectors: a bit cast of a vector
            // element here compiled to the same element for every step)
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const unsigned ka = kq[e], vb = val[e];
              bf16x2 x, y;
              __builtin_memcpy(&x, &ka, 4);
              __builtin_memcpy(&y, &vb, 4);
              d = __builtin_amdgcn_fdot2_f32_bf16(x, y, d, false);
            }
            d = row16_sum(d);  // the row's 16 lanes are one DPP row
            if (valid) {
              if (piece == 0) jbs[NH - 1].rk[relrow(c * CH + row)] = d;
              T* orow = Oseq[h] + (unsigned)((relrow(c * CH + row)) * D + 8 * piece);
              __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(orow));
            }
          } else if (valid) {
            const u32x4 val = *reinterpret_cast<const u32x4*>(sO + TN::off(row, 8 * piece));
            T* orow = Oseq[h] + (unsigned)((relrow(c * CH + row)) * D + 8 * piece);
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(orow));
          }
        }
      }
    };
    if constexpr (OSTAGE && NH == 1) flush_o();

    // ---- state update: S = lambda^cl S + K^T (diag(lambda^(cl-1-j)) V)
    {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const char* const sK = stage + kslot(h) * TB;
#pragma unroll
        for (int tk = 0; tk < NKT; ++tk) accS[h][tk] *= dc;
        op_t Bv[NJS];
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
          if constexpr (E == 8) {
            bf16x8 b;
#pragma unroll
            for (int x = 0; x < 8; ++x) b[x] = (__bf16)((float)Vop[h][js][x] * wv[js][x]);
            Bv[js] = b;
          } else {
            Bv[js] = Vop[h][js] * wv[js][0];
          }
        }
#pragma unroll
        for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
          for (int js = 0; js < NJS; ++js) {
            const op_t Ak = tr_op<T, TN>(sK, js * KS, 16 * tk, lane);
            accS[h][tk] = X::mfma(Ak, Bv[js], accS[h][tk]);
          }
      }
      if (lcf) {
#pragma unroll
        for (int js = 0; js < NJS; ++js)
#pragma unroll
          for (int x = 0; x < E; ++x) wv[js][x] *= lamC;
      }
    }
    if constexpr (OSTAGE && NH == 2) flush_o();
    // ---- DUMP: the state at a boundary row, for callers that need it there
    // (compiled into the walks that may be asked for it only: its mere
    // presence slowed the other walks' chunk loop by a tenth)
    if constexpr (OUT && DUMP) {
      // position after the chunk, counted from the sequence's end when
      // reverse (a sequence has fewer than 2^31 rows: wave-uniform 32-bit
      // scalar arithmetic; a 64-bit remainder here cost about 40 vector
      // instructions per chunk and walk)
      const int pe = (int)t0 + c * CH + cl;
      const int y = jb.reverse ? (int)jb.Ls - pe : pe;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const WalkJob& jh = jbs[h];
        if (jh.dump && y > 0 && y < (int)jb.Ls && (y & ((1 << jh.dump_shift) - 1)) == 0) {
          const int m = y >> jh.dump_shift;
          float* dst = jh.dump + (int64_t)(jh.dump_rev ? jh.ndump - m : m - 1) * D * D;
          // the lane's element offset, formed here: without the empty asm the
          // compiler hoists all NKT x 4 store addresses out of the chunk loop
          // and keeps them in registers the walk needs
          unsigned lo = (unsigned)(4 * g * D + col + l16);
          asm volatile("" : "+v"(lo));
#pragma unroll
          for (int tk = 0; tk < NKT; ++tk)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[lo + (unsigned)((16 * tk + r) * D)] = accS[h][tk][r];
        }
      }
    }
  }

  lds_barrier();  // every wave is done with the last chunk's LDS
  return gsum2 * 0.6931471805599453f;
}

}  // namespace la
