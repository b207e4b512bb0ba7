// One SO(2)-reduced equivariant message-passing layer in the incoming-edge
// layout: forward and backward.
//
// Forward (review of arXiv 2507.03840, "What carries the argument"; MALOQ
// Sec. III, III-C1, III-D, II-B1):
//   rotate_in   per edge: messages n_i (+) n_j rotated into the edge frame by
//               the edge's Wigner rows (|m| <= mmax only), times radial gates
//               -> GEMM operands A_m, one array per |m|
//   GEMMs       Y_m = A_m B_m^T, the SO(2) channel mixing per |m| (MFMA)
//   attention   per destination row: logits from the invariant output
//               channels, softmax over the row (the row is owned, so no
//               exchange is needed)
//   aggregate   per destination row: rotate back, scale by alpha and sum into
//               the destination with a register accumulator (no atomics)
// Backward: the reverse of each step; every reduction over edges runs in a
// fixed order (per-row/per-source waves, split-K partials summed in order).
//
// Data layout in HBM (E = edges, C = channels, nl(m) = lmax - m + 1):
//   A_0 [E][nl(0) * 2C]          column (l) * 2C + slot
//   A_m [E][2 * nl(m) * 2C]      column (sign * nl(m) + l - m) * 2C + slot, sign 0 = +m, 1 = -m
//   Y_0 [E][nl(0) * C], Y_m [E][2 * nl(m) * C]   same pattern with C
// slot 0..C-1 = source channels, C..2C-1 = destination channels.
#include <cstring>
#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "timing.h"

namespace egnn {
namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

template <int LMAX, int MMAX>
struct Lay {
  static constexpr int K = (LMAX + 1) * (LMAX + 1);
  static constexpr int ND = d_count(LMAX, MMAX);
  static constexpr int KEPT = kept_count(LMAX, MMAX);
  static constexpr int NP = pair_count(LMAX, MMAX);
  __host__ __device__ static constexpr int nl(int mu) { return LMAX - mu + 1; }
  __host__ __device__ static constexpr int doff(int l, int m, int mp) {
    return d_block_offset(l, MMAX) + (m + cmin(l, MMAX)) * (2 * l + 1) + (mp + l);
  }
  // column block of kept (l, m) within A_|m| / Y_|m|
  __host__ __device__ static constexpr int col(int l, int m) {
    return m == 0 ? l : ((m > 0 ? 0 : 1) * nl(cabs(m)) + (l - cabs(m)));
  }
  // width of A_mu (in slots of 2C) or Y_mu (in slots of C)
  __host__ __device__ static constexpr int blocks(int mu) { return mu == 0 ? nl(0) : 2 * nl(mu); }
  // running index of kept (l, m)
  __host__ __device__ static constexpr int kidx(int l, int m) {
    int n = 0;
    for (int j = 0; j < l; ++j) n += 2 * cmin(j, MMAX) + 1;
    return n + m + cmin(l, MMAX);
  }
};

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ inline float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ inline float silu(float z) { return z * sigmoidf_(z); }
__device__ inline float dsilu(float z) {
  float s = sigmoidf_(z);
  return s * (1.0f + z * (1.0f - s));
}
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

struct Ptr3 {
  void *p[3];
};
struct CPtr3 {
  const void *p[3];
};

// ---------------------------------------------------------------- weights --
// B_m [2 nl C][2 nl 2C] from W_m1, W_m2 [nl C][nl 2C]:
//   B[+][+] = W_m1, B[+][-] = -W_m2, B[-][+] = W_m2, B[-][-] = W_m1
template <typename TB>
__global__ void expand_weights_kernel(const float *w1, const float *w2, int rows, int cols, TB *B) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = static_cast<int64_t>(4) * rows * cols;
  if (i >= n) return;
  const int k = static_cast<int>(i % (2 * cols));
  const int r = static_cast<int>(i / (2 * cols));
  const int so = r / rows, no = r % rows, si = k / cols, ki = k % cols;
  const int64_t o = static_cast<int64_t>(no) * cols + ki;
  float v = (so == si) ? w1[o] : (so == 0 ? -w2[o] : w2[o]);
  Store<TB>::st(B + i, v);
}

// V2 = a2 W1 + b2 W2, V3 = a3 W1 + b3 W2: the precomputed weight sums of the
// three-product complex GEMM (see gemm.hip).
__global__ void combo_weights_kernel(const float *w1, const float *w2, int64_t n, float a2, float b2, float a3,
                                     float b3, float *v2, float *v3) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  v2[i] = a2 * w1[i] + b2 * w2[i];
  v3[i] = a3 * w1[i] + b3 * w2[i];
}

__global__ void to_bf16_kernel(const float *in, int64_t n, uint16_t *out) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = f32_to_bf16(in[i]);
}

// Radial weights W_rad [n_rbf][np][2C] as bf16 pairs over the basis index:
// out[q][p][j] = (bf16 W[2q][p][j], bf16 W[2q + 1][p][j]) for q < 8, zero past
// n_rbf (the gate of the paired rotate-in is a sum of packed dot products).
__global__ void pack_wrad_kernel(const float *w, int n_rbf, int np, int C2, uint32_t *out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(8) * np * C2) return;
  const int q = static_cast<int>(i / (static_cast<int64_t>(np) * C2));
  const int64_t r = i % (static_cast<int64_t>(np) * C2);
  const float v0 = 2 * q < n_rbf ? w[static_cast<int64_t>(2 * q) * np * C2 + r] : 0.0f;
  const float v1 = 2 * q + 1 < n_rbf ? w[static_cast<int64_t>(2 * q + 1) * np * C2 + r] : 0.0f;
  out[i] = static_cast<uint32_t>(f32_to_bf16(v0)) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
}

// bf16 backward helpers.
// BT[k][n] = B[n][k] in bf16, the second operand of dX = dY B as a product
// with both operands contiguous along its sum (n).  cplx: B is the expanded
// [[W1, -W2], [W2, W1]] of W1, W2 [rows][cols]; else B = W0 [rows][cols].
__global__ void expand_weights_t_kernel(const float *w1, const float *w2, int rows, int cols, bool cplx,
                                        uint16_t *BT) {
  const int R = cplx ? 2 * rows : rows, Cc = cplx ? 2 * cols : cols;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(R) * Cc) return;
  const int k = static_cast<int>(i / R), n = static_cast<int>(i % R);
  float v;
  if (!cplx) {
    v = w1[static_cast<int64_t>(n) * cols + k];
  } else {
    const int so = n / rows, no = n % rows, si = k / cols, ki = k % cols;
    const int64_t o = static_cast<int64_t>(no) * cols + ki;
    v = (so == si) ? w1[o] : (so == 0 ? -w2[o] : w2[o]);
  }
  BT[i] = f32_to_bf16(v);
}

// dW1 = dB(+,+) + dB(-,-) and dW2 = dB(-,+) - dB(+,-) from the gradient dB
// [2 rows][2 cols] of the expanded matrix (the inverse of the expansion).
__global__ void fold_expanded_kernel(const float *dB, int rows, int cols, float *dw1, float *dw2) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(rows) * cols) return;
  const int n = static_cast<int>(i / cols), k = static_cast<int>(i % cols);
  const int64_t ld = 2 * static_cast<int64_t>(cols);
  const float pp = dB[n * ld + k], pm = dB[n * ld + cols + k];
  const float mp = dB[(rows + n) * ld + k], mm = dB[(rows + n) * ld + cols + k];
  dw1[i] = pp + mm;
  dw2[i] = mp - pm;
}

// --------------------------------------------------------------- forward --
// Node-centric edge work.  Every edge's message has a source half (slots
// 0..C-1) and a destination half (slots C..2C-1).  A wave owns one
// (node, half, 64-slot chunk): for half 0 it walks the node's outgoing edges
// (the source grouping), for half 1 its incoming edges (its CSR row).  Either
// way the only node irreps it needs are the node's own row, loaded once, so
// there are no per-edge gathers.  The edges' geometry rows are staged into
// LDS in batches with coalesced vector loads, and the radial weights of the
// wave's slots stay in registers.
constexpr int kBatch = 8;

struct NodeWave {
  int node, half, chunk;
};
__device__ inline NodeWave node_wave(int gw, int nch) {
  NodeWave w;
  const int per_node = 2 * nch;
  w.node = gw / per_node;
  const int r = gw % per_node;
  w.half = r / nch;
  w.chunk = r % nch;
  return w;
}

// Edges of (node, half): half 1 = incoming (row), half 0 = outgoing (source group).
struct EdgeList {
  const int *perm;  // null for a contiguous row
  int begin, count;
  __device__ inline int at(int i) const { return perm ? perm[begin + i] : begin + i; }
};
__device__ inline EdgeList edge_list(int node, int half, int n_dst, const int *row_ptr, const int *src_ptr,
                                     const int *src_perm) {
  EdgeList l;
  if (half == 1) {
    l.perm = nullptr;
    l.begin = node < n_dst ? row_ptr[node] : 0;
    l.count = node < n_dst ? row_ptr[node + 1] - l.begin : 0;
  } else {
    l.perm = src_perm;
    l.begin = src_ptr[node];
    l.count = src_ptr[node + 1] - l.begin;
  }
  l.begin = __builtin_amdgcn_readfirstlane(l.begin);
  l.count = __builtin_amdgcn_readfirstlane(l.count);
  return l;
}

// One channel of a row, in two steps (load, then convert).  bf16: a 16-bit
// load (zero-extended), then one shift into the high half.  (Loading the
// aligned 32-bit word of the channel pair and selecting the lane's half took
// three VALU operations per value.)
template <typename T> struct RawOf { typedef uint32_t type; };
template <> struct RawOf<float> { typedef float type; };
__device__ inline float load_raw(const float *row, uint32_t off) { return row[off]; }
__device__ inline uint32_t load_raw(const uint16_t *row, uint32_t off) { return row[off]; }
__device__ inline float from_raw(float v, uint32_t) { return v; }
__device__ inline float from_raw(uint32_t v, uint32_t) { return __uint_as_float(v << 16); }

// Geometry rows (the first gs4 float4 of each) of a wave's edge list move
// global -> registers -> the wave's LDS buffer in batches of kBatch edges.
// AHEAD: one batch ahead of their use (the loads of batch b + 1 are issued
// before batch b is processed and written to LDS after it), at the price of
// holding that batch in registers meanwhile; otherwise each batch is loaded
// when the previous one is done.  Edge ids (one per lane, a load through
// src_perm for source groups) run one batch ahead either way.  An optional
// per-edge value (extra[e]) rides along into xbuf.  The LDS rows are GS4
// float4 long; the first gs4 hold the row's data.  By default LDS column t is
// float4 column t of the geometry row; a degree part stages two ranges
// instead: NA4 columns from OA4 (its Wigner-D entries), then the columns from
// OB4 (the radial basis values) (see PartCols).
template <int GS4, bool AHEAD = true, bool EXTRA = false, int OA4 = 0, int NA4 = GS4, int OB4 = 0>
struct GeomPipe {
  static constexpr int NQ = (kBatch * GS4 + kWave - 1) / kWave;  // float4 slots per lane
  const EdgeList el;
  typedef float v4 __attribute__((ext_vector_type(4)));  // plain vector: stays in registers
  const v4 *g4;
  const float *extra;
  float4 *buf;
  int *eid;
  float *xbuf;
  int s4, lane, gs4;
  v4 q[NQ];
  // slot u of this lane: edge t / GS4 of the batch, float4 t % GS4 of its row (t = lane + 64 u);
  // columns from gs4 to GS4 - 1 (past the basis values in use) repeat column gs4 - 1
  __device__ int si(int u) const { return (lane + kWave * u) / GS4; }
  __device__ int sq(int u) const {
    const int t = min((lane + kWave * u) % GS4, gs4 - 1);
    if constexpr (NA4 >= GS4 && OA4 == 0)
      return t;
    else
      return t < NA4 ? OA4 + t : OB4 + (t - NA4);
  }
  float xv;
  int ids_cur, ids_next;

  // The loads below carry no branches: past the end of the list they read
  // its last edge again (ids clamp, cnt >= 1) and the results go unused.  A
  // load under a branch makes the compiler copy its result where the paths
  // meet, and that copy waits for every load in flight.
  // this lane's edge id in the batch starting at base (clamped into the list)
  __device__ int batch_edge(int base) const { return el.at(min(base + lane, el.count - 1)); }
  __device__ void fetch(int ids, int cnt) {
    cnt = max(cnt, 1);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      // slots past the batch reload its last row, which commit discards
      const int e = __shfl(ids, min(si(u), cnt - 1), kWave);
      q[u] = g4[static_cast<int64_t>(e) * s4 + sq(u)];
    }
    if constexpr (EXTRA) xv = extra[ids];
  }
  __device__ void commit(int ids, int cnt) {
    if (lane < cnt) {
      eid[lane] = ids;
      if constexpr (EXTRA) xbuf[lane] = xv;
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u)
      if (si(u) < cnt) reinterpret_cast<v4 *>(buf)[lane + kWave * u] = q[u];
  }
  // Loads batch 0 into LDS and starts the ids of batch 1.  el.count > 0.
  __device__ GeomPipe(const EdgeList &el_, const float *geom, int gstride, int gs4_, float4 *buf_, int *eid_,
                      const float *extra_ = nullptr, float *xbuf_ = nullptr)
      : el(el_), g4(reinterpret_cast<const v4 *>(geom)), extra(extra_), buf(buf_), eid(eid_), xbuf(xbuf_),
        s4(gstride / 4), lane(static_cast<int>(threadIdx.x) & (kWave - 1)), gs4(gs4_), xv(0.0f) {
    ids_cur = batch_edge(0);
    const int cnt = min(kBatch, el.count);
    fetch(ids_cur, cnt);
    ids_next = batch_edge(kBatch);
    commit(ids_cur, cnt);
    wave_lds_order();
  }
  __device__ void next_ids(int nb) {
    ids_cur = ids_next;
    ids_next = batch_edge(nb + kBatch);
  }
  // Before processing the batch at base: issue the loads of the next one
  // (AHEAD), or nothing.
  __device__ void prefetch(int base) {
    if constexpr (AHEAD) {
      const int nb = base + kBatch;
      fetch(ids_next, min(kBatch, el.count - nb));
      next_ids(nb);
    }
  }
  // After processing the batch at base: its LDS rows are free; store the next
  // one (loaded now unless AHEAD).
  __device__ void advance(int base) {
    const int nb = base + kBatch;
    wave_lds_order();
    if (nb < el.count) {
      if constexpr (!AHEAD) {
        fetch(ids_next, min(kBatch, el.count - nb));
        next_ids(nb);
      }
      commit(ids_cur, min(kBatch, el.count - nb));
    }
    wave_lds_order();
  }
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Coefficients KB..KB+KR-1 of one channel of a node row (rows of K coefficients).
template <int KR, typename T>
__device__ inline void load_node_range(const T *__restrict__ x, int node, int K, int KB, int C, int c, bool active,
                                       float (&xv)[KR]) {
  const T *row = x + (static_cast<int64_t>(node) * K + KB) * C + (active ? c : 0);
  float v[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) v[k] = Store<T>::ld(row + static_cast<uint32_t>(k * C));
#pragma unroll
  for (int k = 0; k < KR; ++k) xv[k] = active ? v[k] : 0.0f;
}

// Degree parts.  At high degree one wave cannot hold a node's whole
// per-channel state (the radial weights of every gate pair, accumulators for
// every coefficient, the next edge's loads) in registers: the node kernels
// spilled or ran one wave per SIMD.  Their work separates by degree (the
// rotation mixes m only within a degree), so the degrees are dealt to parts,
// each launched as its own grid over the same waves: part p owns degrees
// lo(p)..hi(p), its coefficients, kept entries and gate pairs, and reads
// every edge's geometry again.  Split<LMAX, N> deals 0..LMAX to N parts
// (degrees up to 4 are always one part); each kernel family picks its N.
template <int LMAX, int NP>
struct Split {
  static constexpr int N = LMAX <= 4 ? 1 : NP;
  static_assert(N >= 1 && N <= 4 && (LMAX > 6 || N <= 3), "no such degree split");
  __host__ __device__ static constexpr int lo(int p) {
    return N == 1 ? 0
           : LMAX <= 6 ? (N == 2 ? (p == 0 ? 0 : 4) : (p == 0 ? 0 : p == 1 ? 4 : 6))
           : N == 2    ? (p == 0 ? 0 : 6)
           : N == 3    ? (p == 0 ? 0 : p == 1 ? 5 : 7)
                       : (p == 0 ? 0 : p == 1 ? 4 : p == 2 ? 6 : 8);
  }
  __host__ __device__ static constexpr int hi(int p) { return p == N - 1 ? LMAX : lo(p + 1) - 1; }
};

// Backward node kernels (radial-weight gradient, gather): the split grows
// with the number of radial basis functions, whose weights each lane holds.
template <int LMAX, int NRBF>
using Parts = Split<LMAX, LMAX <= 6 ? (NRBF <= 8 ? 2 : 3) : (NRBF <= 8 ? 3 : 4)>;
// Per-channel rotate-in (it holds the gate weights as well)
template <int LMAX, int NRBF>
using InParts = Split<LMAX, LMAX <= 6 ? (NRBF <= 8 ? 2 : 3) : (NRBF <= 8 ? 3 : 4)>;
// Per-channel aggregate (accumulators and one edge's kept entries only)
template <int LMAX>
using AggParts = Split<LMAX, LMAX <= 6 ? 1 : 2>;
// Row backward at lmax 6 and 8 (bwd_row_dot_kernel, bwd_row_grad_kernel)
template <int LMAX>
using RowParts = Split<LMAX, LMAX <= 6 ? 2 : 3>;

// The geometry columns a degree part stages (GeomPipe): its degrees' Wigner-D
// entries, which sit together in the row (degree-major), and, with NRBF > 0,
// the radial basis values after all of D, each range in whole float4 columns.
// A launch over every degree stages the row's first columns as one range, as
// the single-part kernels always did.  In the LDS row, D entry o is at
// o - DOFF and basis value k at RB + k.
template <int LMAX, int MMAX, int L0, int L1, int NRBF>
struct PartCols {
  static constexpr int ND = d_count(LMAX, MMAX);
  static constexpr bool kWhole = L0 == 0 && L1 == LMAX;
  static constexpr int OA4 = kWhole ? 0 : d_block_offset(L0, MMAX) / 4;
  static constexpr int NA4 = kWhole ? (ND + NRBF + 3) / 4 : (d_block_offset(L1 + 1, MMAX) + 3) / 4 - OA4;
  static constexpr int OB4 = ND / 4;
  static constexpr int DOFF = OA4 * 4;
  static constexpr int RB = kWhole ? ND : NA4 * 4 + ND - OB4 * 4;
  static constexpr int GS4 = kWhole || NRBF == 0 ? NA4 : NA4 + (ND - OB4 * 4 + NRBF + 3) / 4;
  // columns in use for n_rbf basis functions (n_rbf <= NRBF)
  __device__ static int gs4(int n_rbf) {
    return kWhole ? (ND + n_rbf + 3) / 4 : NRBF == 0 ? NA4 : NA4 + (ND - OB4 * 4 + n_rbf + 3) / 4;
  }
};

// Index ranges of degrees L0..L1: coefficients k = l^2 + l + m from KB, kept
// (l, m) entries from QB (their running index), and the gate pairs (m, l)
// with l in the range, numbered m-major from 0.
template <int LMAX, int MMAX, int L0, int L1>
struct Rng {
  static constexpr int KB = L0 * L0;
  static constexpr int KR = (L1 + 1) * (L1 + 1) - KB;
  static constexpr int QB = Lay<LMAX, MMAX>::kidx(L0, -cmin(L0, MMAX));
  static constexpr int QR = Lay<LMAX, MMAX>::kidx(L1, cmin(L1, MMAX)) + 1 - QB;
  __host__ __device__ static constexpr int lpair(int m, int l) {
    int n = 0;
    for (int j = 0; j < m; ++j) {
      const int a = j > L0 ? j : L0;
      if (a <= L1) n += L1 - a + 1;
    }
    return n + l - (m > L0 ? m : L0);
  }
  static constexpr int NP = lpair(MMAX + 1, MMAX + 1 > L0 ? MMAX + 1 : L0);
  // global pair index (pair_index) of local pair q
  __host__ __device__ static constexpr int gpair(int q) {
    for (int m = 0; m <= MMAX; ++m) {
      const int a = m > L0 ? m : L0;
      if (a > L1) continue;
      if (q <= L1 - a) return pair_index(m, a + q, LMAX);
      q -= L1 - a + 1;
    }
    return -1;
  }
};

// Radial weights of the gate pairs of degrees L0..L1 for one lane's slot j
// (unused slots read column 0 and are zeroed after: no branch per load).
template <int LMAX, int MMAX, int NRBF, int L0, int L1>
__device__ inline void load_wrad_range(const float *wrad, int n_rbf, int C2, int j, bool active,
                                       float (&wr)[NRBF][Rng<LMAX, MMAX, L0, L1>::NP]) {
  using R = Rng<LMAX, MMAX, L0, L1>;
  constexpr int NPG = pair_count(LMAX, MMAX);
  const int jc = active ? j : 0;
  float v[NRBF][R::NP];
#pragma unroll
  for (int k = 0; k < NRBF; ++k)
#pragma unroll
    for (int m = 0; m <= MMAX; ++m)
#pragma unroll
      for (int l = (m > L0 ? m : L0); l <= L1; ++l)
        v[k][R::lpair(m, l)] = wrad[(static_cast<int64_t>(k < n_rbf ? k : 0) * NPG + pair_index(m, l, LMAX)) * C2 + jc];
#pragma unroll
  for (int k = 0; k < NRBF; ++k)
#pragma unroll
    for (int p = 0; p < R::NP; ++p) wr[k][p] = (active && k < n_rbf) ? v[k][p] : 0.0f;
}

// The same as bf16 pairs over the basis index (k = 2q, 2q + 1), rounded as
// pack_wrad_kernel rounds them, for the bf16-storage rotate-in: its gate then
// takes NRBF / 2 packed dot products (v_dot2_f32_bf16, fp32 accumulate) per
// pair, with half the registers of the fp32 form.
template <int LMAX, int MMAX, int NRBF, int L0, int L1>
__device__ inline void load_wrad_bf16_range(const float *wrad, int n_rbf, int C2, int j, bool active,
                                            bf16x2 (&wp)[NRBF / 2][Rng<LMAX, MMAX, L0, L1>::NP]) {
  using R = Rng<LMAX, MMAX, L0, L1>;
  float v[NRBF][R::NP];
  load_wrad_range<LMAX, MMAX, NRBF, L0, L1>(wrad, n_rbf, C2, j, active, v);
#pragma unroll
  for (int q = 0; q < NRBF / 2; ++q)
#pragma unroll
    for (int p = 0; p < R::NP; ++p) wp[q][p] = bf16x2{static_cast<__bf16>(v[2 * q][p]), static_cast<__bf16>(v[2 * q + 1][p])};
}

// A[e] = g_e * trunc(D_e x) for the wave's half of every edge of its node
// (degrees L0..L1 of it: one degree part).
template <int LMAX, int MMAX, int NRBF, typename T, typename TA, int L0 = 0, int L1 = LMAX>
__global__ void __launch_bounds__(kThreads) scatter_in_kernel(const int *__restrict__ row_ptr,
                                                              const int *__restrict__ src_ptr,
                                                              const int *__restrict__ src_perm,
                                                              const float *__restrict__ geom, int gstride, int n_dst,
                                                              int n_src, const T *__restrict__ x, int C,
                                                              const float *__restrict__ wrad, int n_rbf, Ptr3 A) {
  using L = Lay<LMAX, MMAX>;
  using R = Rng<LMAX, MMAX, L0, L1>;  // this launch's degrees
  using P = PartCols<LMAX, MMAX, L0, L1, NRBF>;  // and their geometry columns
  constexpr int GS4 = P::GS4;
  const int gs4 = P::gs4(n_rbf);
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nch = (C + kWave - 1) / kWave;
  const NodeWave nw = node_wave(blockIdx.x * kWavesPerBlock + wave, nch);
  if (nw.node >= n_src) return;
  const EdgeList el = edge_list(nw.node, nw.half, n_dst, row_ptr, src_ptr, src_perm);
  if (el.count == 0) return;
  const int C2 = 2 * C;
  const int c = nw.chunk * kWave + lane;
  const bool active = c < C;
  const int j = nw.half * C + c;
  float xv[R::KR];  // the node row's degrees L0..L1
  load_node_range<R::KR>(x, nw.node, L::K, R::KB, C, c, active, xv);
  // fp32 storage: fp32 radial weights; bf16 storage: bf16 pairs (see load_wrad_bf16_range)
  constexpr bool kPacked = std::is_same<TA, uint16_t>::value;
  float wr[kPacked ? 1 : NRBF][kPacked ? 1 : R::NP];
  bf16x2 wp[kPacked ? NRBF / 2 : 1][kPacked ? R::NP : 1];
  if constexpr (kPacked)
    load_wrad_bf16_range<LMAX, MMAX, NRBF, L0, L1>(wrad, n_rbf, C2, j, active, wp);
  else
    load_wrad_range<LMAX, MMAX, NRBF, L0, L1>(wrad, n_rbf, C2, j, active, wr);
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  // bf16: fewer registers for higher occupancy instead of the batch ahead
  GeomPipe<GS4, std::is_same<T, float>::value, false, P::OA4, P::NA4, P::OB4> gp(el, geom, gstride, gs4, gbuf[wave],
                                                                                eids[wave]);
  for (int base = 0; base < el.count; base += kBatch) {
    const int cnt = min(kBatch, el.count - base);
    gp.prefetch(base);
    for (int i = 0; i < cnt; ++i) {
      const int e = uniform(eids[wave][i]);
      const float *gr = gb + i * GS4 * 4;
      float g[R::NP];
#pragma unroll
      for (int p = 0; p < R::NP; ++p) g[p] = 0.0f;
      if constexpr (kPacked) {
#pragma unroll
        for (int q = 0; q < NRBF / 2; ++q) {
          // basis slots past n_rbf hold finite copies (GeomPipe) and meet zero
          // weights, so they add nothing: no select or branch per basis function
          const float r0 = gr[P::RB + 2 * q], r1 = gr[P::RB + 2 * q + 1];
          const bf16x2 ph{static_cast<__bf16>(r0), static_cast<__bf16>(r1)};
#pragma unroll
          for (int p = 0; p < R::NP; ++p) g[p] = __builtin_amdgcn_fdot2_f32_bf16(ph, wp[q][p], g[p], false);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NRBF; ++k) {
          // (slots past n_rbf: finite values times zero weights)
          const float ph = gr[P::RB + k];
#pragma unroll
          for (int p = 0; p < R::NP; ++p) g[p] += ph * wr[k][p];
        }
      }
      if (!active) continue;
      // wave-uniform row pointers; the lane offsets below stay 32-bit
      TA *rowp[MMAX + 1];
#pragma unroll
      for (int mu = 0; mu <= MMAX; ++mu)
        rowp[mu] = static_cast<TA *>(A.p[mu]) + static_cast<int64_t>(e) * (L::blocks(mu) * C2);
#pragma unroll
      for (int l = L0; l <= L1; ++l) {
#pragma unroll
        for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
          float v = 0.0f;
#pragma unroll
          for (int mp = -l; mp <= l; ++mp) v += gr[L::doff(l, m, mp) - P::DOFF] * xv[l * l + l + mp - R::KB];
          v *= g[R::lpair(cabs(m), l)];
          Store<TA>::st(rowp[cabs(m)] + static_cast<uint32_t>(L::col(l, m) * C2 + j), v);
        }
      }
    }
    gp.advance(base);
  }
}

// bf16 storage, C a multiple of 128: as scatter_in_kernel with two adjacent
// channels per lane (a wave covers 128 channels).  Each Wigner-D value read
// from LDS feeds both channels, the node row and the radial weights come in as
// channel pairs, and each output leaves as one packed conversion and one
// 4-byte store.
template <int LMAX, int MMAX, int NRBF>
__global__ void __launch_bounds__(kThreads) scatter_in_pair_kernel(const int *__restrict__ row_ptr,
                                                                   const int *__restrict__ src_ptr,
                                                                   const int *__restrict__ src_perm,
                                                                   const float *__restrict__ geom, int gstride,
                                                                   int n_dst, int n_src,
                                                                   const uint16_t *__restrict__ x, int C,
                                                                   const uint32_t *__restrict__ wpk, int n_rbf, Ptr3 A) {
  using L = Lay<LMAX, MMAX>;
  constexpr int GS4 = (L::ND + NRBF + 3) / 4;
  constexpr int NP = L::NP;
  const int gs4 = (L::ND + n_rbf + 3) / 4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nch = C / (2 * kWave);
  const NodeWave nw = node_wave(blockIdx.x * kWavesPerBlock + wave, nch);
  if (nw.node >= n_src) return;
  const EdgeList el = edge_list(nw.node, nw.half, n_dst, row_ptr, src_ptr, src_perm);
  if (el.count == 0) return;
  const int C2 = 2 * C;
  const int c = nw.chunk * 2 * kWave + 2 * lane;  // channels c, c + 1 (always < C)
  const int j = nw.half * C + c;
  // the node row, both channels: one 32-bit load per coefficient
  float xv[L::K][2];
  {
    const uint32_t *row = reinterpret_cast<const uint32_t *>(x + static_cast<int64_t>(nw.node) * L::K * C + c);
    uint32_t raw[L::K];
#pragma unroll
    for (int k = 0; k < L::K; ++k) raw[k] = row[k * (C / 2)];
#pragma unroll
    for (int k = 0; k < L::K; ++k) {
      xv[k][0] = __uint_as_float(raw[k] << 16);
      xv[k][1] = __uint_as_float(raw[k] & 0xFFFF0000u);
    }
  }
  // radial weights of both slots, pre-packed as bf16 pairs over the basis index (pack_wrad_kernel)
  bf16x2 wp[2][NRBF / 2][NP];
#pragma unroll
  for (int q = 0; q < NRBF / 2; ++q)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint2 w = *reinterpret_cast<const uint2 *>(wpk + (static_cast<int64_t>(q) * NP + p) * C2 + j);
      wp[0][q][p] = __builtin_bit_cast(bf16x2, w.x);
      wp[1][q][p] = __builtin_bit_cast(bf16x2, w.y);
    }
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  GeomPipe<GS4, false> gp(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
  for (int base = 0; base < el.count; base += kBatch) {
    const int cnt = min(kBatch, el.count - base);
    gp.prefetch(base);
    for (int i = 0; i < cnt; ++i) {
      const int e = uniform(eids[wave][i]);
      const float *gr = gb + i * GS4 * 4;
      bf16x2 ph[NRBF / 2];
#pragma unroll
      for (int q = 0; q < NRBF / 2; ++q) {
        // (slots past n_rbf: finite values times the zero weights pack_wrad_kernel wrote)
        const float r0 = gr[L::ND + 2 * q], r1 = gr[L::ND + 2 * q + 1];
        ph[q] = bf16x2{static_cast<__bf16>(r0), static_cast<__bf16>(r1)};
      }
      uint32_t *rowp[MMAX + 1];  // wave-uniform row bases; 32-bit lane offsets below
#pragma unroll
      for (int mu = 0; mu <= MMAX; ++mu)
        rowp[mu] = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(A.p[mu]) + static_cast<int64_t>(e) * (L::blocks(mu) * C2));
      // pair by pair: the gate of (|m|, l), then its +m and -m rows
#pragma unroll
      for (int mu = 0; mu <= MMAX; ++mu)
#pragma unroll
        for (int l = mu; l <= LMAX; ++l) {
          const int pi = pair_index(mu, l, LMAX);
          float g0 = 0.0f, g1 = 0.0f;
#pragma unroll
          for (int q = 0; q < NRBF / 2; ++q) {
            g0 = __builtin_amdgcn_fdot2_f32_bf16(ph[q], wp[0][q][pi], g0, false);
            g1 = __builtin_amdgcn_fdot2_f32_bf16(ph[q], wp[1][q][pi], g1, false);
          }
#pragma unroll
          for (int sg = 0; sg < (mu == 0 ? 1 : 2); ++sg) {
            const int m = sg == 0 ? mu : -mu;
            float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
            for (int mp = -l; mp <= l; ++mp) {
              const float d = gr[L::doff(l, m, mp)];
              v0 += d * xv[l * l + l + mp][0];
              v1 += d * xv[l * l + l + mp][1];
            }
            const bf16x2 out{static_cast<__bf16>(v0 * g0), static_cast<__bf16>(v1 * g1)};
            rowp[mu][static_cast<uint32_t>((L::col(l, m) * C2 + j) / 2)] = __builtin_bit_cast(uint32_t, out);
          }
        }
    }
    gp.advance(base);
  }
}

// Logits and softmax over one destination row per wave.  Sixteen lanes share
// an edge (16-byte loads of its invariant output plane, reduced with four
// butterfly steps), so four edges are read per pass with coalesced rows.
// Lane 16g keeps a running (max, sum) over the edges it owns; the row's
// softmax combines them in a fixed order, and the same lanes write alpha.
template <typename T>
__global__ void __launch_bounds__(kThreads) attention_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                             const T *__restrict__ Y0, int ldy0, int C,
                                                             const float *__restrict__ w_att, float *logit,
                                                             float *alpha) {
  constexpr int VW = 16 / sizeof(T);  // channels per 16-byte load
  constexpr int U = 4;                // edge groups in flight per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int d = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (d >= n_dst) return;
  const int b = row_ptr[d], end = row_ptr[d + 1];
  if (b == end) return;
  const int grp = lane >> 4, sub = lane & 15;
  float M = -INFINITY, S = 0.0f;
  for (int base = b; base < end; base += 4 * U) {
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.0f;
    for (int c0 = sub * VW; c0 < C; c0 += 16 * VW) {  // one chunk per lane up to 16 VW channels
      // every group's load before any use; past the row's end the last edge is
      // read again and its sum not used (no branch around the loads)
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = min(base + 4 * u + grp, end - 1);
        raw[u] = *reinterpret_cast<const uint4 *>(Y0 + static_cast<int64_t>(e) * ldy0 + c0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        T v[VW];
        memcpy(v, &raw[u], sizeof(raw[u]));
#pragma unroll
        for (int j = 0; j < VW; ++j) acc[u] += w_att[c0 + j] * silu(Store<T>::ld(&v[j]));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = acc[u];
      a += __shfl_xor(a, 8);
      a += __shfl_xor(a, 4);
      a += __shfl_xor(a, 2);
      a += __shfl_xor(a, 1);
      const int e = base + 4 * u + grp;
      if (sub == 0 && e < end) {
        logit[e] = a;
        const float Mn = fmaxf(M, a);
        S = S * expf(M - Mn) + expf(a - Mn);
        M = Mn;
      }
    }
  }
  const float Mrow = wave_max(M);
  const float Srow = wave_sum(M == -INFINITY ? 0.0f : S * expf(M - Mrow));
  const float inv = 1.0f / Srow;
  // the row's logits were stored by the sub == 0 lanes; the waves of a block
  // share the CU's vector cache, so a block-scope fence makes them visible to
  // every lane of the wave, and all lanes share the last pass
  __threadfence_block();
  for (int e = b + lane; e < end; e += kWave) alpha[e] = expf(logit[e] - Mrow) * inv;
}

// x_out[d] = x[d] + sum_e alpha_e D_e^T Yhat_e ; edge_out[e] = D_e^T Yhat_e.
// One wave per (destination row, 64-channel chunk): it walks the row's
// contiguous edges, staging their geometry rows (and alpha) into LDS in
// batches; the accumulator stays in registers (no atomics, no partials).
// Degrees L0..L1 only (one degree part: see Parts).
template <int LMAX, int MMAX, typename T, int L0 = 0, int L1 = LMAX>
__global__ void __launch_bounds__(kThreads) aggregate_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                             const float *__restrict__ geom, int gstride, int nd_rbf,
                                                             const float *__restrict__ alpha, CPtr3 Y, int C,
                                                             const T *__restrict__ x, T *__restrict__ x_out,
                                                             T *__restrict__ edge_out) {
  using L = Lay<LMAX, MMAX>;
  using R = Rng<LMAX, MMAX, L0, L1>;  // this launch's degrees
  using P = PartCols<LMAX, MMAX, L0, L1, 0>;  // and their Wigner-D columns
  constexpr int GS4 = P::GS4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  __shared__ float abuf[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nch = (C + kWave - 1) / kWave;
  const int gw = uniform(blockIdx.x * kWavesPerBlock + wave);
  const int d = gw / nch, chunk = gw % nch;
  if (d >= n_dst) return;
  const int c = chunk * kWave + lane;
  const bool on = c < C;
  const int cl = on ? c : C - 1;  // clamped channel for loads
  EdgeList el;
  el.perm = nullptr;
  el.begin = uniform(row_ptr[d]);
  el.count = uniform(row_ptr[d + 1]) - el.begin;
  (void)nd_rbf;
  float acc[R::KR];
#pragma unroll
  for (int k = 0; k < R::KR; ++k) acc[k] = 0.0f;
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  if (el.count > 0) {
    // not ahead: each edge's Y loads follow at once and wait for the geometry in any case
    GeomPipe<GS4, false, true, P::OA4, P::NA4> gp(el, geom, gstride, GS4, gbuf[wave], eids[wave], alpha, abuf[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp.prefetch(base);
      for (int i = 0; i < cnt; ++i) {
        const int e = el.begin + base + i;
        const float a = abuf[wave][i];
        const float *gr = gb + i * GS4 * 4;
        float y[R::QR];
#pragma unroll
        for (int l = L0; l <= L1; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            const int mu = cabs(m);
            const T *row = static_cast<const T *>(Y.p[mu]) + static_cast<int64_t>(e) * L::blocks(mu) * C;
            y[L::kidx(l, m) - R::QB] = Store<T>::ld(row + L::col(l, m) * C + cl);
          }
        T *eo = edge_out ? edge_out + static_cast<int64_t>(e) * L::K * C : nullptr;
#pragma unroll
        for (int l = L0; l <= L1; ++l)
#pragma unroll
          for (int mp = -l; mp <= l; ++mp) {
            float msg = 0.0f;
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
              msg += gr[L::doff(l, m, mp) - P::DOFF] * y[L::kidx(l, m) - R::QB];
            acc[l * l + l + mp - R::KB] += a * msg;
            if (eo && on) Store<T>::st(eo + (l * l + l + mp) * C + c, msg);
          }
      }
      gp.advance(base);
    }
  }
  if (!on) return;
#pragma unroll
  for (int k = 0; k < R::KR; ++k) {
    const int64_t o = (static_cast<int64_t>(d) * L::K + R::KB + k) * C + c;
    Store<T>::st(x_out + o, Store<T>::ld(x + o) + acc[k]);
  }
}

// bf16 storage, C a multiple of 128: as aggregate_kernel with two adjacent
// channels per lane (one 32-bit load per Y entry, each Wigner-D value used
// for both channels, packed bf16 stores).
template <int LMAX, int MMAX>
__global__ void __launch_bounds__(kThreads) aggregate_pair_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                                  const float *__restrict__ geom, int gstride,
                                                                  const float *__restrict__ alpha, CPtr3 Y, int C,
                                                                  const uint16_t *__restrict__ x,
                                                                  uint16_t *__restrict__ x_out,
                                                                  uint16_t *__restrict__ edge_out) {
  using L = Lay<LMAX, MMAX>;
  constexpr int GS4 = (L::ND + 3) / 4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  __shared__ float abuf[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nch = C / (2 * kWave);
  const int gw = uniform(blockIdx.x * kWavesPerBlock + wave);
  const int d = gw / nch, chunk = gw % nch;
  if (d >= n_dst) return;
  const int c = chunk * 2 * kWave + 2 * lane;  // channels c, c + 1 (always < C)
  EdgeList el;
  el.perm = nullptr;
  el.begin = uniform(row_ptr[d]);
  el.count = uniform(row_ptr[d + 1]) - el.begin;
  float acc[L::K][2];
#pragma unroll
  for (int k = 0; k < L::K; ++k) acc[k][0] = acc[k][1] = 0.0f;
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  auto unpack = [](uint32_t v, float &lo, float &hi) {
    lo = __uint_as_float(v << 16);
    hi = __uint_as_float(v & 0xFFFF0000u);
  };
  auto pack = [](float lo, float hi) { return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(lo), static_cast<__bf16>(hi)}); };
  if (el.count > 0) {
    GeomPipe<GS4, false, true> gp(el, geom, gstride, (L::ND + 3) / 4, gbuf[wave], eids[wave], alpha, abuf[wave]);
    // The row's Y rows are contiguous, so the next edge's loads go out before
    // this edge's products across batch boundaries too (j indexes the row's
    // edges; two named buffers, two edges per round, the last round repeating
    // an edge's loads): 4.13 -> 4.08 ms over three GeSbTe layers.
    auto load_y = [&](int j, uint32_t(&yr)[L::KEPT]) {
      const int e = el.begin + min(j, el.count - 1);
#pragma unroll
      for (int l = 0; l <= LMAX; ++l)
#pragma unroll
        for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
          const int mu = cabs(m);
          const uint32_t *row = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(Y.p[mu]) +
                                                                   static_cast<int64_t>(e) * L::blocks(mu) * C);
          yr[L::kidx(l, m)] = row[static_cast<uint32_t>((L::col(l, m) * C + c) / 2)];
        }
    };
    auto product = [&](int j, const uint32_t(&yr)[L::KEPT]) {
      const int i = j % kBatch;  // the edge's slot in the staged batch
      const int e = el.begin + j;
      const float a = abuf[wave][i];
      const float *gr = gb + i * GS4 * 4;
      uint32_t *eo = edge_out ? reinterpret_cast<uint32_t *>(edge_out + static_cast<int64_t>(e) * L::K * C) : nullptr;
#pragma unroll
      for (int l = 0; l <= LMAX; ++l)
#pragma unroll
        for (int mp = -l; mp <= l; ++mp) {
          float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            const float dv = gr[L::doff(l, m, mp)];
            float y0, y1;
            unpack(yr[L::kidx(l, m)], y0, y1);
            m0 += dv * y0;
            m1 += dv * y1;
          }
          acc[l * l + l + mp][0] += a * m0;
          acc[l * l + l + mp][1] += a * m1;
          if (eo) eo[static_cast<uint32_t>(((l * l + l + mp) * C + c) / 2)] = pack(m0, m1);
        }
    };
    static_assert(kBatch % 2 == 0, "a pair of edges never straddles two batches");
    uint32_t ya[L::KEPT], yb[L::KEPT];
    load_y(0, ya);
    for (int j = 0; j < el.count; j += 2) {
      if (j > 0 && j % kBatch == 0) gp.advance(j - kBatch);  // stage the batch that starts at j
      load_y(j + 1, yb);
      product(j, ya);
      load_y(j + 2, ya);
      if (j + 1 < el.count) product(j + 1, yb);
    }
  }
  const uint32_t *xr = reinterpret_cast<const uint32_t *>(x + static_cast<int64_t>(d) * L::K * C + c);
  uint32_t *xo = reinterpret_cast<uint32_t *>(x_out + static_cast<int64_t>(d) * L::K * C + c);
#pragma unroll
  for (int k = 0; k < L::K; ++k) {
    float x0, x1;
    unpack(xr[k * (C / 2)], x0, x1);
    xo[k * (C / 2)] = pack(x0 + acc[k][0], x1 + acc[k][1]);
  }
}

// -------------------------------------------------------------- backward --
// Per destination row: T_e = trunc(D_e G_d); dalpha_e = <Y_e, T_e>;
// da_e = alpha_e (dalpha_e - sum_row alpha dalpha);
// dY_e = alpha_e T_e + da_e w_att SiLU'(Y_e[0,0]) on (l=0, m=0);
// w_att partial of the row = sum_e da_e SiLU(Y_e[0,0]).
// One wave per row; lanes = channels (CPL per lane), geometry rows staged in
// LDS in batches as in the forward aggregate.
template <int LMAX, int MMAX, int CPL, typename TY, typename TD>
__global__ void __launch_bounds__(kThreads) bwd_row_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                           const float *__restrict__ geom, int gstride,
                                                           const float *__restrict__ alpha, CPtr3 Y, int C,
                                                           const float *__restrict__ G, const float *__restrict__ w_att,
                                                           Ptr3 dY, float *dalpha, float *watt_part) {
  using L = Lay<LMAX, MMAX>;
  constexpr int GS4 = (L::ND + 3) / 4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int d = uniform(blockIdx.x * kWavesPerBlock + wave);
  if (d >= n_dst) return;
  EdgeList el;
  el.perm = nullptr;
  el.begin = uniform(row_ptr[d]);
  el.count = uniform(row_ptr[d + 1]) - el.begin;
  const int gs4 = (L::ND + 3) / 4;
  float gd[CPL][L::K];
  int cl[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int c = lane + kWave * t;
    cl[t] = c < C ? c : C - 1;
#pragma unroll
    for (int k = 0; k < L::K; ++k) gd[t][k] = c < C ? G[(static_cast<int64_t>(d) * L::K + k) * C + c] : 0.0f;
  }
  auto edge_T = [&](const float *gr, int t, float (&T)[L::KEPT]) {
#pragma unroll
    for (int l = 0; l <= LMAX; ++l)
#pragma unroll
      for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
        float v = 0.0f;
#pragma unroll
        for (int mp = -l; mp <= l; ++mp) v += gr[L::doff(l, m, mp)] * gd[t][l * l + l + mp];
        T[L::kidx(l, m)] = v;
      }
  };
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  float s_row = 0.0f;
  float wacc[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) wacc[t] = 0.0f;
  if (el.count > 0) {
    GeomPipe<GS4> gp(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp.prefetch(base);
      for (int i = 0; i < cnt; ++i) {
        const int e = el.begin + base + i;
        const float *gr = gb + i * GS4 * 4;
        float p = 0.0f;
        // all of the edge's Y loads before any use (see load_raw)
        typename RawOf<TY>::type yr[CPL][L::KEPT];
#pragma unroll
        for (int t = 0; t < CPL; ++t)
#pragma unroll
          for (int l = 0; l <= LMAX; ++l)
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
              const int mu = cabs(m);
              const TY *row = static_cast<const TY *>(Y.p[mu]) + static_cast<int64_t>(e) * L::blocks(mu) * C;
              yr[t][L::kidx(l, m)] = load_raw(row, static_cast<uint32_t>(L::col(l, m) * C + cl[t]));
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          float T[L::KEPT];
          edge_T(gr, t, T);
#pragma unroll
          for (int l = 0; l <= LMAX; ++l)
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
              // gd is 0 on clamped lanes, so T is too
              p += from_raw(yr[t][L::kidx(l, m)], static_cast<uint32_t>(L::col(l, m) * C + cl[t])) * T[L::kidx(l, m)];
        }
        p = wave_sum(p);
        dalpha[e] = p;  // every lane stores the same value and later reads its own store
        s_row += alpha[e] * p;
      }
      gp.advance(base);
    }
    GeomPipe<GS4> gp2(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp2.prefetch(base);
      for (int i = 0; i < cnt; ++i) {
        const int e = el.begin + base + i;
        const float *gr = gb + i * GS4 * 4;
        const float a = alpha[e];
        const float da = a * (dalpha[e] - s_row);
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          const int c = lane + kWave * t;
          float T[L::KEPT];
          edge_T(gr, t, T);
          const float y00 = Store<TY>::ld(static_cast<const TY *>(Y.p[0]) + static_cast<int64_t>(e) * L::blocks(0) * C + cl[t]);
          const float wat = w_att[cl[t]];
#pragma unroll
          for (int l = 0; l <= LMAX; ++l)
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
              float v = a * T[L::kidx(l, m)];
              if (l == 0) {
                v += da * wat * dsilu(y00);
                if (c < C) wacc[t] += da * silu(y00);
              }
              const int mu = cabs(m);
              TD *row = static_cast<TD *>(dY.p[mu]) + static_cast<int64_t>(e) * L::blocks(mu) * C;
              if (c < C) Store<TD>::st(row + static_cast<uint32_t>(L::col(l, m) * C + c), v);
            }
        }
      }
      gp2.advance(base);
    }
  }
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int c = lane + kWave * t;
    if (c < C) watt_part[static_cast<int64_t>(d) * C + c] = wacc[t];
  }
}

// The row backward in degree parts (lmax 6 and 8, where one wave cannot hold
// G_d and an edge's kept entries for every degree and channel slot).  The dot
// dalpha_e sums over degrees, so it is built in part order: part 0 writes its
// share, each later part adds its own (bwd_row_dot_kernel).  Then each part
// forms its degrees' dY from the finished dalpha (bwd_row_grad_kernel); the
// part holding degree 0 also adds the attention term and writes the w_att
// partial.  Same waves, lanes and staging as bwd_row_kernel; each part stages
// only its degrees' Wigner-D columns.
template <int LMAX, int MMAX, int CPL, typename TY, int L0, int L1>
__global__ void __launch_bounds__(kThreads) bwd_row_dot_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                               const float *__restrict__ geom, int gstride, CPtr3 Y,
                                                               int C, const float *__restrict__ G,
                                                               float *__restrict__ dalpha) {
  using L = Lay<LMAX, MMAX>;
  using R = Rng<LMAX, MMAX, L0, L1>;
  using P = PartCols<LMAX, MMAX, L0, L1, 0>;
  constexpr int GS4 = P::GS4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int d = uniform(blockIdx.x * kWavesPerBlock + wave);
  if (d >= n_dst) return;
  EdgeList el;
  el.perm = nullptr;
  el.begin = uniform(row_ptr[d]);
  el.count = uniform(row_ptr[d + 1]) - el.begin;
  if (el.count == 0) return;
  float gd[CPL][R::KR];
  int cl[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) {
    const int c = lane + kWave * t;
    cl[t] = c < C ? c : C - 1;
#pragma unroll
    for (int k = 0; k < R::KR; ++k)
      gd[t][k] = c < C ? G[(static_cast<int64_t>(d) * L::K + R::KB + k) * C + c] : 0.0f;
  }
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  GeomPipe<GS4, true, false, P::OA4, P::NA4> gp(el, geom, gstride, GS4, gbuf[wave], eids[wave]);
  for (int base = 0; base < el.count; base += kBatch) {
    const int cnt = min(kBatch, el.count - base);
    gp.prefetch(base);
    for (int i = 0; i < cnt; ++i) {
      const int e = el.begin + base + i;
      const float *gr = gb + i * GS4 * 4;
      // all of the edge's Y loads before any use (see load_raw)
      typename RawOf<TY>::type yr[CPL][R::QR];
#pragma unroll
      for (int t = 0; t < CPL; ++t)
#pragma unroll
        for (int l = L0; l <= L1; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            const int mu = cabs(m);
            const TY *row = static_cast<const TY *>(Y.p[mu]) + static_cast<int64_t>(e) * L::blocks(mu) * C;
            yr[t][L::kidx(l, m) - R::QB] = load_raw(row, static_cast<uint32_t>(L::col(l, m) * C + cl[t]));
          }
      const float prev = L0 == 0 ? 0.0f : dalpha[e];
      __builtin_amdgcn_sched_barrier(0);
      float p = 0.0f;
#pragma unroll
      for (int t = 0; t < CPL; ++t)
#pragma unroll
        for (int l = L0; l <= L1; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            float v = 0.0f;  // T(l, m); gd is 0 on clamped lanes, so T is too
#pragma unroll
            for (int mp = -l; mp <= l; ++mp) v += gr[L::doff(l, m, mp) - P::DOFF] * gd[t][l * l + l + mp - R::KB];
            p += from_raw(yr[t][L::kidx(l, m) - R::QB], static_cast<uint32_t>(L::col(l, m) * C + cl[t])) * v;
          }
      p = wave_sum(p);
      dalpha[e] = prev + p;  // every lane stores the same value
    }
    gp.advance(base);
  }
}

template <int LMAX, int MMAX, int CPL, typename TY, typename TD, int L0, int L1>
__global__ void __launch_bounds__(kThreads) bwd_row_grad_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                                const float *__restrict__ geom, int gstride,
                                                                const float *__restrict__ alpha, CPtr3 Y, int C,
                                                                const float *__restrict__ G,
                                                                const float *__restrict__ w_att, Ptr3 dY,
                                                                const float *__restrict__ dalpha,
                                                                float *__restrict__ watt_part) {
  using L = Lay<LMAX, MMAX>;
  using R = Rng<LMAX, MMAX, L0, L1>;
  using P = PartCols<LMAX, MMAX, L0, L1, 0>;
  constexpr int GS4 = P::GS4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int d = uniform(blockIdx.x * kWavesPerBlock + wave);
  if (d >= n_dst) return;
  EdgeList el;
  el.perm = nullptr;
  el.begin = uniform(row_ptr[d]);
  el.count = uniform(row_ptr[d + 1]) - el.begin;
  float wacc[CPL];
#pragma unroll
  for (int t = 0; t < CPL; ++t) wacc[t] = 0.0f;
  if (el.count > 0) {
    float gd[CPL][R::KR];
    int cl[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + kWave * t;
      cl[t] = c < C ? c : C - 1;
#pragma unroll
      for (int k = 0; k < R::KR; ++k)
        gd[t][k] = c < C ? G[(static_cast<int64_t>(d) * L::K + R::KB + k) * C + c] : 0.0f;
    }
    // sum over the row of alpha dalpha: lanes over edges, then the wave (the same value in every part)
    float s = 0.0f;
    for (int i = lane; i < el.count; i += kWave) s += alpha[el.begin + i] * dalpha[el.begin + i];
    const float s_row = wave_sum(s);
    const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
    GeomPipe<GS4, true, false, P::OA4, P::NA4> gp(el, geom, gstride, GS4, gbuf[wave], eids[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp.prefetch(base);
      for (int i = 0; i < cnt; ++i) {
        const int e = el.begin + base + i;
        const float *gr = gb + i * GS4 * 4;
        const float a = alpha[e];
        const float da = a * (dalpha[e] - s_row);
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          const int c = lane + kWave * t;
          float y00 = 0.0f, wat = 0.0f;
          if constexpr (L0 == 0) {
            y00 = Store<TY>::ld(static_cast<const TY *>(Y.p[0]) + static_cast<int64_t>(e) * L::blocks(0) * C + cl[t]);
            wat = w_att[cl[t]];
          }
#pragma unroll
          for (int l = L0; l <= L1; ++l)
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
              float T = 0.0f;
#pragma unroll
              for (int mp = -l; mp <= l; ++mp) T += gr[L::doff(l, m, mp) - P::DOFF] * gd[t][l * l + l + mp - R::KB];
              float v = a * T;
              if (l == 0) {
                v += da * wat * dsilu(y00);
                if (c < C) wacc[t] += da * silu(y00);
              }
              const int mu = cabs(m);
              TD *row = static_cast<TD *>(dY.p[mu]) + static_cast<int64_t>(e) * L::blocks(mu) * C;
              if (c < C) Store<TD>::st(row + static_cast<uint32_t>(L::col(l, m) * C + c), v);
            }
        }
      }
      gp.advance(base);
    }
  }
  if constexpr (L0 == 0) {
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + kWave * t;
      if (c < C) watt_part[static_cast<int64_t>(d) * C + c] = wacc[t];
    }
  }
}

// ------------------------------------------------------- edge-update block --
// e_out[e] = e_in[e] + D_e^T Yhat_e: the node block's per-edge message added to
// the edge embedding instead of being aggregated.  One wave per edge (grid
// stride), lanes over channels; the edge's Wigner rows are staged in LDS and
// read as broadcasts.  e_out may be e_in: a lane reads its entries of the edge
// before it writes them.
template <int LMAX, int MMAX, int CPL, typename T>
__global__ void __launch_bounds__(kThreads) edge_update_kernel(int64_t E, const float *__restrict__ geom, int gstride,
                                                               CPtr3 Y, int C, const T *e_in, T *e_out) {
  using L = Lay<LMAX, MMAX>;
  __shared__ float dsm[kWavesPerBlock][L::ND];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; e < E;
       e += static_cast<int64_t>(gridDim.x) * kWavesPerBlock) {
    const float *gr = geom + e * gstride;
    for (int i = lane; i < L::ND; i += kWave) dsm[wave][i] = gr[i];
    wave_lds_order();
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + kWave * t;
      if (c < C) {
        float y[L::KEPT], ev[L::K];
#pragma unroll
        for (int l = 0; l <= LMAX; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            const int mu = cabs(m);
            const T *row = static_cast<const T *>(Y.p[mu]) + e * L::blocks(mu) * C;
            y[L::kidx(l, m)] = Store<T>::ld(row + L::col(l, m) * C + c);
          }
        const T *ei = e_in + e * L::K * C + c;
#pragma unroll
        for (int k = 0; k < L::K; ++k) ev[k] = Store<T>::ld(ei + k * C);
        T *eo = e_out + e * L::K * C + c;
#pragma unroll
        for (int l = 0; l <= LMAX; ++l)
#pragma unroll
          for (int mp = -l; mp <= l; ++mp) {
            float v = ev[l * l + l + mp];
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) v += dsm[wave][L::doff(l, m, mp)] * y[L::kidx(l, m)];
            Store<T>::st(eo + (l * l + l + mp) * C, v);
          }
      }
    }
    wave_lds_order();
  }
}

// Backward of the edge-update block, first step: dY_e = trunc(D_e dE_e), in
// the layout of Y and the storage type (TD), for the shared SO(2) backward.
template <int LMAX, int MMAX, int CPL, typename TD>
__global__ void __launch_bounds__(kThreads) edge_dy_kernel(int64_t E, const float *__restrict__ geom, int gstride,
                                                           const float *__restrict__ dE, int C, Ptr3 dY) {
  using L = Lay<LMAX, MMAX>;
  __shared__ float dsm[kWavesPerBlock][L::ND];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; e < E;
       e += static_cast<int64_t>(gridDim.x) * kWavesPerBlock) {
    const float *gr = geom + e * gstride;
    for (int i = lane; i < L::ND; i += kWave) dsm[wave][i] = gr[i];
    wave_lds_order();
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + kWave * t;
      if (c < C) {
        float de[L::K];
        const float *di = dE + e * L::K * C + c;
#pragma unroll
        for (int k = 0; k < L::K; ++k) de[k] = di[k * C];
#pragma unroll
        for (int l = 0; l <= LMAX; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            float v = 0.0f;
#pragma unroll
            for (int mp = -l; mp <= l; ++mp) v += dsm[wave][L::doff(l, m, mp)] * de[l * l + l + mp];
            const int mu = cabs(m);
            TD *row = static_cast<TD *>(dY.p[mu]) + e * L::blocks(mu) * C;
            Store<TD>::st(row + L::col(l, m) * C + c, v);
          }
      }
    }
    wave_lds_order();
  }
}

// Radial-weight gradient: dW_rad[k][p][j] = sum_e phi_e[k] dg_e[p][j] with
// dg_e[p] = sum_{+-m} dX_e[l,+-m] * Xt_e[l,+-m] (Xt = edge-frame input before
// the gate).  Node-centric waves as in scatter_in; wave (node, half, chunk)
// recomputes Xt of its half from its node's row.  Each wave walks a strided
// stream of nodes and keeps its partial sums in registers; partials are
// written per stream and summed later in a fixed order.
// bwd_row for bf16 storage and C = 2 * 64: lane i owns channels 2i and 2i + 1,
// so Y and dY move as packed pairs (one 32-bit access per entry instead of two
// 16-bit ones), and each rotated entry is formed for both channels from the
// same geometry value and used at once, with no per-channel array of T kept.
template <int LMAX, int MMAX>
__global__ void __launch_bounds__(kThreads) bwd_row_pair_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                                const float *__restrict__ geom, int gstride,
                                                                const float *__restrict__ alpha, CPtr3 Y, int C,
                                                                const float *__restrict__ G,
                                                                const float *__restrict__ w_att, Ptr3 dY,
                                                                float *dalpha, float *watt_part) {
  using L = Lay<LMAX, MMAX>;
  constexpr int GS4 = (L::ND + 3) / 4;
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int d = uniform(blockIdx.x * kWavesPerBlock + wave);
  if (d >= n_dst) return;
  EdgeList el;
  el.perm = nullptr;
  el.begin = uniform(row_ptr[d]);
  el.count = uniform(row_ptr[d + 1]) - el.begin;
  const int gs4 = (L::ND + 3) / 4;
  const int c = 2 * lane;
  float gd[L::K][2];
#pragma unroll
  for (int k = 0; k < L::K; ++k) {
    const float2 g = *reinterpret_cast<const float2 *>(G + (static_cast<int64_t>(d) * L::K + k) * C + c);
    gd[k][0] = g.x;
    gd[k][1] = g.y;
  }
  auto unpack = [](uint32_t v, float &lo, float &hi) {
    lo = __uint_as_float(v << 16);
    hi = __uint_as_float(v & 0xFFFF0000u);
  };
  auto pack = [](float lo, float hi) { return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(lo), static_cast<__bf16>(hi)}); };
  // entry (l, m) of T_e = trunc(D_e G_d) for both channels
  auto entry = [&](const float *gr, int l, int m, float &v0, float &v1) {
    v0 = v1 = 0.0f;
#pragma unroll
    for (int mp = -l; mp <= l; ++mp) {
      const float dv = gr[L::doff(l, m, mp)];
      v0 += dv * gd[l * l + l + mp][0];
      v1 += dv * gd[l * l + l + mp][1];
    }
  };
  auto yrow = [&](int e, int mu) {
    return reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(Y.p[mu]) +
                                              static_cast<int64_t>(e) * L::blocks(mu) * C);
  };
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  float s_row = 0.0f, wacc0 = 0.0f, wacc1 = 0.0f;
  if (el.count > 0) {
    GeomPipe<GS4> gp(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp.prefetch(base);
      for (int i = 0; i < cnt; ++i) {
        const int e = el.begin + base + i;
        const float *gr = gb + i * GS4 * 4;
        // all of the edge's Y loads before any use (see load_raw)
        uint32_t yr[L::KEPT];
#pragma unroll
        for (int l = 0; l <= LMAX; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
            yr[L::kidx(l, m)] = yrow(e, cabs(m))[static_cast<uint32_t>((L::col(l, m) * C + c) / 2)];
        __builtin_amdgcn_sched_barrier(0);
        float p = 0.0f;
#pragma unroll
        for (int l = 0; l <= LMAX; ++l) {
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            float v0, v1, y0, y1;
            entry(gr, l, m, v0, v1);
            unpack(yr[L::kidx(l, m)], y0, y1);
            p += y0 * v0 + y1 * v1;
          }
          // one degree's geometry at a time in registers
          __builtin_amdgcn_sched_barrier(0);
        }
        p = wave_sum(p);
        dalpha[e] = p;  // every lane stores the same value and later reads its own store
        s_row += alpha[e] * p;
      }
      gp.advance(base);
    }
    const float2 wat = *reinterpret_cast<const float2 *>(w_att + c);
    GeomPipe<GS4> gp2(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp2.prefetch(base);
      for (int i = 0; i < cnt; ++i) {
        const int e = el.begin + base + i;
        const float *gr = gb + i * GS4 * 4;
        const float a = alpha[e];
        const float da = a * (dalpha[e] - s_row);
        float y00, y01;
        unpack(yrow(e, 0)[static_cast<uint32_t>((L::col(0, 0) * C + c) / 2)], y00, y01);
#pragma unroll
        for (int l = 0; l <= LMAX; ++l) {
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            float v0, v1;
            entry(gr, l, m, v0, v1);
            v0 *= a;
            v1 *= a;
            if (l == 0) {
              v0 += da * wat.x * dsilu(y00);
              v1 += da * wat.y * dsilu(y01);
              wacc0 += da * silu(y00);
              wacc1 += da * silu(y01);
            }
            const int mu = cabs(m);
            uint32_t *row = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(dY.p[mu]) +
                                                         static_cast<int64_t>(e) * L::blocks(mu) * C);
            row[static_cast<uint32_t>((L::col(l, m) * C + c) / 2)] = pack(v0, v1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      gp2.advance(base);
    }
  }
  *reinterpret_cast<float2 *>(watt_part + static_cast<int64_t>(d) * C + c) = make_float2(wacc0, wacc1);
}



template <int LMAX, int MMAX, int NRBF, typename T, int L0 = 0, int L1 = LMAX>
__global__ void __launch_bounds__(kThreads) wrad_grad_kernel(const int *__restrict__ row_ptr,
                                                             const int *__restrict__ src_ptr,
                                                             const int *__restrict__ src_perm,
                                                             const float *__restrict__ geom, int gstride, int n_dst,
                                                             int n_src, const T *__restrict__ x, int C, int n_rbf,
                                                             CPtr3 dA, int n_streams, float *__restrict__ part) {
  using L = Lay<LMAX, MMAX>;
  using R = Rng<LMAX, MMAX, L0, L1>;  // this launch's degrees
  using P = PartCols<LMAX, MMAX, L0, L1, NRBF>;  // and their geometry columns
  constexpr int GS4 = P::GS4;
  const int gs4 = P::gs4(n_rbf);
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nch = (C + kWave - 1) / kWave;
  const int per_node = 2 * nch;
  const int gw = uniform(blockIdx.x * kWavesPerBlock + wave);
  if (gw >= n_streams * per_node) return;
  const int stream = gw / per_node, r = gw % per_node;
  const int half = r / nch, chunk = r % nch;
  const int C2 = 2 * C;
  const int c = chunk * kWave + lane;
  const bool active = c < C;
  const int j = half * C + c;
  float acc[NRBF][R::NP];
#pragma unroll
  for (int k = 0; k < NRBF; ++k)
#pragma unroll
    for (int p = 0; p < R::NP; ++p) acc[k][p] = 0.0f;
  const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
  for (int node = stream; node < n_src; node += n_streams) {
    const EdgeList el = edge_list(node, half, n_dst, row_ptr, src_ptr, src_perm);
    if (el.count == 0) continue;
    float xv[R::KR];  // the node row's degrees L0..L1
    load_node_range<R::KR>(x, node, L::K, R::KB, C, c, active, xv);
    GeomPipe<GS4, true, false, P::OA4, P::NA4, P::OB4> gp(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
    for (int base = 0; base < el.count; base += kBatch) {
      const int cnt = min(kBatch, el.count - base);
      gp.prefetch(base);
      // the next edge's dA loads go out before this edge's products (two named
      // buffers, two edges per round, as in gather_grad_kernel); idle lanes
      // load a clamped channel and their sums are never written
      using Raw = typename RawOf<T>::type;
      const int jl = half * C + min(c, C - 1);
      auto load_da = [&](int i, Raw(&raw)[R::QR]) {
        const int e = uniform(eids[wave][min(i, cnt - 1)]);
        const T *rowp[MMAX + 1];  // wave-uniform row bases, 32-bit lane offsets; dA in the storage type
#pragma unroll
        for (int mu = 0; mu <= MMAX; ++mu)
          rowp[mu] = static_cast<const T *>(dA.p[mu]) + static_cast<int64_t>(e) * (L::blocks(mu) * C2);
#pragma unroll
        for (int l = L0; l <= L1; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
            raw[L::kidx(l, m) - R::QB] = load_raw(rowp[cabs(m)], static_cast<uint32_t>(L::col(l, m) * C2 + jl));
      };
      auto product = [&](int i, const Raw(&raw)[R::QR]) {
        const float *gr = gb + i * GS4 * 4;
        float dg[R::NP];
#pragma unroll
        for (int p = 0; p < R::NP; ++p) dg[p] = 0.0f;
#pragma unroll
        for (int l = L0; l <= L1; ++l)
#pragma unroll
          for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m) {
            float xt = 0.0f;
#pragma unroll
            for (int mp = -l; mp <= l; ++mp) xt += gr[L::doff(l, m, mp) - P::DOFF] * xv[l * l + l + mp - R::KB];
            const float dx = from_raw(raw[L::kidx(l, m) - R::QB], static_cast<uint32_t>(L::col(l, m) * C2 + jl));
            dg[R::lpair(cabs(m), l)] += dx * xt;
          }
#pragma unroll
        for (int k = 0; k < NRBF; ++k) {
          // in the staged row (finite); sums of slots past n_rbf are never written
          const float ph = gr[P::RB + k];
#pragma unroll
          for (int p = 0; p < R::NP; ++p) acc[k][p] += ph * dg[p];
        }
      };
      if constexpr (NRBF > 8) {  // 16 radial functions: no registers for a second buffer
        for (int i = 0; i < cnt; ++i) {
          Raw ra[R::QR];
          load_da(i, ra);
          __builtin_amdgcn_sched_barrier(0);
          product(i, ra);
        }
      } else {
        Raw ra[R::QR], rb[R::QR];
        load_da(0, ra);
        for (int i = 0; i < cnt; i += 2) {
          load_da(i + 1, rb);
          product(i, ra);
          load_da(i + 2, ra);
          if (i + 1 < cnt) product(i + 1, rb);
        }
      }
      gp.advance(base);
    }
  }
  if (!active) return;
#pragma unroll
  for (int k = 0; k < NRBF; ++k)
#pragma unroll
    for (int q = 0; q < R::NP; ++q)
      if (k < n_rbf) part[((static_cast<int64_t>(stream) * n_rbf + k) * L::NP + R::gpair(q)) * C2 + j] = acc[k][q];
}

// grad_x[n] = G[n] (owned rows; none when G is null) + sum over the node's incoming edges of
// D_e^T (g_e * dX_e)[destination half] + sum over its outgoing edges of
// D_e^T (g_e * dX_e)[source half], with dX the GEMM gradient of the gated
// edge-frame input.  The waves of one node (two halves x channel chunks) sit
// in one block and their partial sums are added through LDS in a fixed order.
// PK: the gates come from the radial weights packed as bf16 pairs over the
// basis index and the basis values rounded to bf16 pairs, by the same packed
// dot products as the paired rotate-in, so they are the gates that forward used.
template <int LMAX, int MMAX, int NRBF, typename TdA, bool PK = false, int L0 = 0, int L1 = LMAX>
__global__ void __launch_bounds__(kThreads) gather_grad_kernel(const int *__restrict__ row_ptr,
                                                               const int *__restrict__ src_ptr,
                                                               const int *__restrict__ src_perm,
                                                               const float *__restrict__ geom, int gstride, int n_dst,
                                                               int n_src, int C, const float *__restrict__ wrad,
                                                               const uint32_t *__restrict__ wpk, int n_rbf, CPtr3 dA,
                                                               const float *__restrict__ G, float *__restrict__ gx) {
  using L = Lay<LMAX, MMAX>;
  using R = Rng<LMAX, MMAX, L0, L1>;  // this launch's degrees
  using P = PartCols<LMAX, MMAX, L0, L1, NRBF>;  // and their geometry columns
  constexpr int GS4 = P::GS4;
  const int gs4 = P::gs4(n_rbf);
  __shared__ float4 gbuf[kWavesPerBlock][kBatch * GS4];
  __shared__ int eids[kWavesPerBlock][kBatch];
  __shared__ float red[kWavesPerBlock][R::KR * kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nch = (C + kWave - 1) / kWave;
  const NodeWave nw = node_wave(blockIdx.x * kWavesPerBlock + wave, nch);
  const bool live = nw.node < n_src;
  const int C2 = 2 * C;
  const int c = nw.chunk * kWave + lane;
  const bool active = live && c < C;
  const int j = nw.half * C + c;
  float acc[R::KR];
#pragma unroll
  for (int k = 0; k < R::KR; ++k) acc[k] = 0.0f;
  if (live) {
    const EdgeList el = edge_list(nw.node, nw.half, n_dst, row_ptr, src_ptr, src_perm);
    float wr[PK ? 1 : NRBF][R::NP];
    bf16x2 wp[PK ? NRBF / 2 : 1][R::NP];
    if constexpr (PK) {
#pragma unroll
      for (int q = 0; q < NRBF / 2; ++q)
#pragma unroll
        for (int m = 0; m <= MMAX; ++m)
#pragma unroll
          for (int l = (m > L0 ? m : L0); l <= L1; ++l)
            wp[q][R::lpair(m, l)] = __builtin_bit_cast(
                bf16x2, wpk[(static_cast<int64_t>(q) * L::NP + pair_index(m, l, LMAX)) * C2 + (active ? j : 0)]);
    } else {
      load_wrad_range<LMAX, MMAX, NRBF, L0, L1>(wrad, n_rbf, C2, j, active, wr);
    }
    const float *gb = reinterpret_cast<const float *>(gbuf[wave]);
    if (el.count > 0) {
      GeomPipe<GS4, true, false, P::OA4, P::NA4, P::OB4> gp(el, geom, gstride, gs4, gbuf[wave], eids[wave]);
      for (int base = 0; base < el.count; base += kBatch) {
        const int cnt = min(kBatch, el.count - base);
        gp.prefetch(base);
        // the next edge's dA loads go out before this edge's products: two named
        // buffers, two edges per round (the last round repeats an edge's loads
        // and skips its products).  Idle lanes load a clamped channel and their
        // sums are never written.
        using Raw = typename RawOf<TdA>::type;
        const int jl = nw.half * C + min(c, C - 1);
        auto load_da = [&](int i, Raw(&raw)[R::QR]) {
          const int e = uniform(eids[wave][min(i, cnt - 1)]);
          const TdA *rowp[MMAX + 1];  // wave-uniform row bases, 32-bit lane offsets
#pragma unroll
          for (int mu = 0; mu <= MMAX; ++mu)
            rowp[mu] = static_cast<const TdA *>(dA.p[mu]) + static_cast<int64_t>(e) * (L::blocks(mu) * C2);
#pragma unroll
          for (int l = L0; l <= L1; ++l)
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
              raw[L::kidx(l, m) - R::QB] = load_raw(rowp[cabs(m)], static_cast<uint32_t>(L::col(l, m) * C2 + jl));
        };
        auto product = [&](int i, const Raw(&raw)[R::QR]) {
          const float *gr = gb + i * GS4 * 4;
          float dxt[R::QR];
#pragma unroll
          for (int q = 0; q < R::QR; ++q) dxt[q] = from_raw(raw[q], 0u);
          float g[R::NP];
#pragma unroll
          for (int p = 0; p < R::NP; ++p) g[p] = 0.0f;
          if constexpr (PK) {
#pragma unroll
            for (int q = 0; q < NRBF / 2; ++q) {
              const float r0 = gr[P::RB + 2 * q], r1 = gr[P::RB + 2 * q + 1];
              // (slots past n_rbf: finite values times zero weights)
              const bf16x2 ph = {static_cast<__bf16>(r0), static_cast<__bf16>(r1)};
#pragma unroll
              for (int p = 0; p < R::NP; ++p) g[p] = __builtin_amdgcn_fdot2_f32_bf16(ph, wp[q][p], g[p], false);
            }
          } else {
#pragma unroll
            for (int kk = 0; kk < NRBF; ++kk) {
              const float ph = gr[P::RB + kk];  // (slots past n_rbf: finite values times zero weights)
#pragma unroll
              for (int p = 0; p < R::NP; ++p) g[p] += ph * wr[kk][p];
            }
          }
          // gated entries h = g dxt once per (l, m), then one FMA per Wigner-D term
          float h[R::QR];
#pragma unroll
          for (int l = L0; l <= L1; ++l)
#pragma unroll
            for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
              h[L::kidx(l, m) - R::QB] = g[R::lpair(cabs(m), l)] * dxt[L::kidx(l, m) - R::QB];
#pragma unroll
          for (int l = L0; l <= L1; ++l)
#pragma unroll
            for (int mp = -l; mp <= l; ++mp) {
              float sum = 0.0f;
#pragma unroll
              for (int m = -cmin(l, MMAX); m <= cmin(l, MMAX); ++m)
                sum += gr[L::doff(l, m, mp) - P::DOFF] * h[L::kidx(l, m) - R::QB];
              acc[l * l + l + mp - R::KB] += sum;
            }
        };
        if constexpr (NRBF > 8) {  // 16 radial functions: no registers for a second buffer
          for (int i = 0; i < cnt; ++i) {
            Raw ra[R::QR];
            load_da(i, ra);
            __builtin_amdgcn_sched_barrier(0);
            product(i, ra);
          }
        } else {
          Raw ra[R::QR], rb[R::QR];
          load_da(0, ra);
          for (int i = 0; i < cnt; i += 2) {
            load_da(i + 1, rb);
            product(i, ra);
            load_da(i + 2, ra);
            if (i + 1 < cnt) product(i + 1, rb);
          }
        }
        gp.advance(base);
      }
    }
  }
  // half 1 hands its partial to half 0 of the same chunk
#pragma unroll
  for (int k = 0; k < R::KR; ++k) red[wave][k * kWave + lane] = acc[k];
  __syncthreads();
  if (active && nw.half == 0) {
    const int partner = wave + nch;  // same node, same chunk, half 1
#pragma unroll
    for (int k = 0; k < R::KR; ++k) {
      const int64_t o = (static_cast<int64_t>(nw.node) * L::K + R::KB + k) * C + c;
      const float g0 = (G && nw.node < n_dst) ? G[o] : 0.0f;  // no G: the edge block has no node residual
      gx[o] = g0 + (acc[k] + red[partner][k * kWave + lane]);
    }
  }
}

// out[c] = sum_{r < R} in[r*ld + c] in a fixed order (4 row-strided partials, then a fixed tree).
__global__ void __launch_bounds__(256) colsum_kernel(const float *__restrict__ in, int R, int64_t ncol, int64_t ld,
                                                     float *__restrict__ out) {
  __shared__ float part[4][64];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + cx;
  float s = 0.0f;
  if (c < ncol)
    for (int r = ry; r < R; r += 4) s += in[static_cast<int64_t>(r) * ld + c];
  part[ry][cx] = s;
  __syncthreads();
  if (ry == 0 && c < ncol) out[c] = (part[0][cx] + part[1][cx]) + (part[2][cx] + part[3][cx]);
}

// colsum_kernel on four adjacent columns per thread (16-byte loads and
// stores; the same order of sums for every column).  nq = ncol / 4, ld a
// multiple of 4, in and out 16-byte aligned.
__global__ void __launch_bounds__(256) colsum4_kernel(const float *__restrict__ in, int R, int64_t nq, int64_t ld,
                                                      float *__restrict__ out) {
  __shared__ float4 part[4][64];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 64 + cx;
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (q < nq)
    for (int r = ry; r < R; r += 4) {
      const float4 v = reinterpret_cast<const float4 *>(in + static_cast<int64_t>(r) * ld)[q];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
  part[ry][cx] = s;
  __syncthreads();
  if (ry == 0 && q < nq) {
    const float4 a = part[0][cx], b = part[1][cx], c = part[2][cx], d = part[3][cx];
    reinterpret_cast<float4 *>(out)[q] =
        make_float4((a.x + b.x) + (c.x + d.x), (a.y + b.y) + (c.y + d.y), (a.z + b.z) + (c.z + d.z),
                    (a.w + b.w) + (c.w + d.w));
  }
}

// out[c] = sum_{r < R} in[r*ld + c] in a fixed order (four columns per thread where the layout allows)
void colsum(const float *in, int R, int64_t ncol, int64_t ld, float *out, hipStream_t st) {
  const bool quad = ncol % 4 == 0 && ld % 4 == 0 && (reinterpret_cast<uintptr_t>(in) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  if (quad)
    colsum4_kernel<<<ceil_div(ncol / 4, 64), 256, 0, st>>>(in, R, ncol / 4, ld, out);
  else
    colsum_kernel<<<ceil_div(ncol, 64), 256, 0, st>>>(in, R, ncol, ld, out);
}

// Rows [y RB, min(R, (y + 1) RB)) of the 64 columns of block x, summed in the
// order of colsum_kernel, to out[y][c].
__global__ void __launch_bounds__(256) colsum_chunk_kernel(const float *__restrict__ in, int R, int RB, int64_t ncol,
                                                           int64_t ld, float *__restrict__ out) {
  __shared__ float part[4][64];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + cx;
  const int r0 = blockIdx.y * RB, r1 = min(R, r0 + RB);
  float s = 0.0f;
  if (c < ncol)
    for (int r = r0 + ry; r < r1; r += 4) s += in[static_cast<int64_t>(r) * ld + c];
  part[ry][cx] = s;
  __syncthreads();
  if (ry == 0 && c < ncol) out[static_cast<int64_t>(blockIdx.y) * ncol + c] = (part[0][cx] + part[1][cx]) + (part[2][cx] + part[3][cx]);
}

// out[c] = sum_{r < R} in[r*ld + c] in a fixed order.  Many rows over few
// columns would leave most of the GPU idle while a few threads walk every
// row, so rows are first summed in chunks of 64 by blocks of their own (the
// chunk sums go to scratch, ceil(R / 64) * ncol floats), then the chunk sums.
void colsum_fixed(const float *in, int R, int64_t ncol, int64_t ld, float *out, float *scratch, int64_t scratch_floats,
                  hipStream_t st) {
  constexpr int RB = 64;
  const int nchunk = (R + RB - 1) / RB;
  if (R <= RB || static_cast<int64_t>(nchunk) * ncol > scratch_floats) {
    colsum(in, R, ncol, ld, out, st);
    return;
  }
  colsum_chunk_kernel<<<dim3(ceil_div(ncol, 64), nchunk), 256, 0, st>>>(in, R, RB, ncol, ld, scratch);
  colsum(scratch, nchunk, ncol, ncol, out, st);
}

__global__ void fill_f32(float *p, int64_t n, float v) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------ buffers --
size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

inline bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

struct Carver {
  char *base;
  size_t off = 0;
  template <typename T>
  T *take(size_t count) {
    T *r = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += a256(count * sizeof(T));
    return r;
  }
};

struct Acts {  // what the backward needs from the forward
  void *A[3];
  void *Y[3];      // fp32, or bf16 when the storage is bf16
  float *alpha;
};

Acts carve_acts(Carver &cv, const LayerShape &s, int64_t E) {
  Acts a{};
  const size_t ab = s.storage == EGNN_BF16 ? 2 : 4;
  for (int m = 0; m <= s.mmax; ++m) {
    a.A[m] = cv.take<char>(static_cast<size_t>(E) * s.Kg[m] * ab);
  }
  for (int m = 0; m <= s.mmax; ++m) a.Y[m] = cv.take<char>(static_cast<size_t>(E) * s.Ng[m] * ab);
  a.alpha = cv.take<float>(E);
  return a;
}

struct FwdWs {
  void *B[3];      // expanded weights per m (B[0] may alias W0 for fp32)
  float *logit;
  uint32_t *wpk;   // bf16: radial weights packed for the paired rotate-in (pack_wrad_kernel)
};

FwdWs carve_fwd_ws(Carver &cv, const LayerShape &s, int64_t E) {
  FwdWs w{};
  const size_t bb = s.storage == EGNN_BF16 ? 2 : 4;
  for (int m = 0; m <= s.mmax; ++m) {
    if (m == 0 && s.storage == EGNN_F32) {
      w.B[0] = nullptr;
      continue;
    }
    // bf16: expanded [[W1, -W2], [W2, W1]]; fp32 (m >= 1): V2 and V3 of the complex GEMM
    const size_t n = s.storage == EGNN_BF16 ? static_cast<size_t>(s.Ng[m]) * s.Kg[m]
                                             : static_cast<size_t>(s.Ng[m]) * s.Kg[m] / 2;
    w.B[m] = cv.take<char>(n * bb);
  }
  w.logit = cv.take<float>(E);
  w.wpk = s.storage == EGNN_BF16 ? cv.take<uint32_t>(static_cast<size_t>(8) * s.n_pairs * 2 * s.C) : nullptr;
  return w;
}

// Split-K count of the weight-gradient GEMMs (K = edges); a multiple of 8
// from 8 up, so each XCD takes the same number of splits.
int dw_splits(int64_t E) {
  int64_t s = E / 8192;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  if (s >= 8) s = s / 8 * 8;
  return static_cast<int>(s);
}

// Split count of one weight-gradient product with `tiles` output tiles and
// `per_split` partial floats per split, for a kernel of which a CU holds `occ`
// workgroups, on XCDs of `cus` CUs.  The bounds: at most 128 splits, at least
// 2048 edges per split, within the partial buffer sized for dw_splits(E)
// splits of the largest product (`cap_floats`).  Below 8 splits: dw_splits(E),
// raised toward ~1024 blocks in all.  From 8 up the count is 8 q: split z runs
// on XCD z % 8, so each XCD runs q * tiles equal blocks of E / (8 q) edges on
// its CUs; the busiest CU runs ceil(q * tiles / cus) of them, and the product
// takes time in proportion to ceil(q * tiles / cus) / q.  q minimises that
// among the q that keep min(3, occ) blocks per CU on average (with fewer the
// products wait on memory), ties to fewer splits (fewer partials to sum).
// On the 25-tile fp32 m = 0 product of the HfO2 step, splits 16, 32, 48, 56
// and 64 took 2.85, 2.57, 2.18, 2.23 and 2.34 ms, in line with this.
int dw_splits_for(int64_t E, int tiles, int64_t per_split, int64_t cap_floats, int occ, int cus) {
  int64_t s = dw_splits(E);
  tiles = tiles > 0 ? tiles : 1;
  int64_t want = (1024 + tiles - 1) / tiles;
  want = want < 128 ? want : 128;
  const int64_t by_edges = E / 2048, by_buffer = per_split > 0 ? cap_floats / per_split : s;
  if (want > by_edges) want = by_edges;
  if (want > by_buffer) want = by_buffer;
  if (want > s) s = want;
  if (s < 8) return static_cast<int>(s < 1 ? 1 : s);
  int64_t hi = 128;
  if (hi > by_edges) hi = by_edges;
  if (hi > by_buffer) hi = by_buffer;
  const int64_t q_hi = hi / 8 > 0 ? hi / 8 : 1;
  cus = cus > 0 ? cus : 1;
  const int64_t need = static_cast<int64_t>(occ < 3 ? (occ > 0 ? occ : 1) : 3) * cus;
  int64_t q_lo = (need + tiles - 1) / tiles;
  if (q_lo > q_hi) q_lo = q_hi;
  int64_t best = q_lo, best_busy = (q_lo * tiles + cus - 1) / cus;
  for (int64_t q = q_lo + 1; q <= q_hi; ++q) {
    const int64_t busy = (q * tiles + cus - 1) / cus;
    if (busy * best < best_busy * q) {  // busy / q < best_busy / best
      best = q;
      best_busy = busy;
    }
  }
  return static_cast<int>(8 * best);
}

struct BwdWs {
  float *B[3];       // fp32: V2, V3 of the conjugate complex product (m >= 1)
  float *dY[3];      // fp32 storage
  uint16_t *BT[3];   // bf16: transposed (expanded) weights of dX = dY B
  uint16_t *dYb[3];  // bf16 storage: dY in bf16
  float *dA[3];      // fp32 storage
  uint16_t *dAb[3];  // bf16 storage: dA in bf16
  float *dalpha;
  float *watt_part;
  float *P;          // split partials (real and imaginary parts for m >= 1)
  int64_t P_floats;  // its size
  float *wrad_part;
  float *dWexp;        // bf16: summed gradient of the expanded weight of one |m|
  uint32_t *wpk;       // bf16: radial weights packed as in the forward (pack_wrad_kernel)
};

// bf16 layers whose rotate-in runs on channel pairs, with the radial weights
// packed once per call as bf16 pairs (16 basis functions would spill there,
// and so would degree 8).  Every bf16 rotate-in forms its gates from bf16
// radial weights and basis values by packed dot products (the per-channel
// kernel converts the weights itself, with the same rounding), and the
// backward node gradient of every bf16 layer takes its gates the same way.
inline bool paired_gates(const LayerShape &s) {
  return s.storage == EGNN_BF16 && s.C % (2 * kWave) == 0 && s.n_rbf <= 8 && s.lmax <= 6;
}

// node streams of the radial-weight gradient (fixed by the node count, so the
// summation order of its partials is reproducible)
int wrad_streams(int n_src) { return n_src < 1024 ? (n_src > 0 ? n_src : 1) : 1024; }

BwdWs carve_bwd_ws(Carver &cv, const LayerShape &s, int64_t E, int n_dst, int n_src) {
  BwdWs w{};
  const bool bf = s.storage == EGNN_BF16;
  size_t pmax = 0;
  for (int m = 0; m <= s.mmax; ++m) {
    const size_t ng = s.Ng[m], kg = s.Kg[m];
    if (bf) {
      w.BT[m] = cv.take<uint16_t>(ng * kg);
      w.dYb[m] = cv.take<uint16_t>(static_cast<size_t>(E) * ng);
    } else {
      w.B[m] = m == 0 ? nullptr : cv.take<float>(ng * kg / 2);
      w.dY[m] = cv.take<float>(static_cast<size_t>(E) * ng);
    }
    if (bf)
      w.dAb[m] = cv.take<uint16_t>(static_cast<size_t>(E) * kg);
    else
      w.dA[m] = cv.take<float>(static_cast<size_t>(E) * kg);
    pmax = pmax > ng * kg ? pmax : ng * kg;
  }
  w.dalpha = cv.take<float>(E);
  w.watt_part = cv.take<float>(static_cast<size_t>(n_dst > 0 ? n_dst : 1) * s.C);
  w.P = cv.take<float>(pmax * dw_splits(E));
  w.P_floats = static_cast<int64_t>(pmax) * dw_splits(E);
  w.wrad_part = cv.take<float>(static_cast<size_t>(wrad_streams(n_src)) * s.n_rbf * s.n_pairs * 2 * s.C);
  if (bf) w.dWexp = cv.take<float>(pmax);
  w.wpk = bf ? cv.take<uint32_t>(static_cast<size_t>(8) * s.n_pairs * 2 * s.C) : nullptr;
  return w;
}

struct WOff {  // offsets of the packed weight blocks
  size_t W0, W1[3], W2[3], wrad, watt, total;
};
WOff weight_offsets(const LayerShape &s) {
  WOff o{};
  size_t p = 0;
  o.W0 = p;
  p += static_cast<size_t>(s.Ng[0]) * s.Kg[0];
  for (int m = 1; m <= s.mmax; ++m) {
    size_t blk = static_cast<size_t>(s.Ng[m] / 2) * (s.Kg[m] / 2);
    o.W1[m] = p;
    p += blk;
    o.W2[m] = p;
    p += blk;
  }
  o.wrad = p;
  p += static_cast<size_t>(s.n_rbf) * s.n_pairs * 2 * s.C;
  o.watt = p;
  p += s.C;
  o.total = p;
  return o;
}

// ------------------------------------------------------------ launchers --
// f(lo, hi) for each part of the degree split S in order, lo and hi as
// integral constants
template <typename S, int P = 0, typename F>
void for_parts(F &&f) {
  if constexpr (P < S::N) {
    f(std::integral_constant<int, S::lo(P)>{}, std::integral_constant<int, S::hi(P)>{});
    for_parts<S, P + 1>(f);
  }
}

template <int LMAX, int MMAX>
struct Launch {
  template <typename T, typename TA>
  static void rotate_in(const egnn_graph *g, const LayerShape &s, const float *geom, const T *x, const float *wrad,
                        const uint32_t *wpk, const Acts &a, hipStream_t st) {
    Ptr3 A{{a.A[0], a.A[1], a.A[2]}};
    // channel pairs up to degree 6 (paired_gates): at degree 8 the pair
    // kernel's node row and radial weights for two channels spill, and the
    // per-channel kernel with fp32 radial weights runs instead
    if constexpr (std::is_same<T, uint16_t>::value && std::is_same<TA, uint16_t>::value && LMAX <= 6) {
      if (wpk && paired_gates(s)) {  // channel pairs
        const int nch2 = s.C / (2 * kWave);
        const unsigned grid2 = ceil_div(static_cast<int64_t>(g->n_src) * 2 * nch2, kWavesPerBlock);
        scatter_in_pair_kernel<LMAX, MMAX, 8><<<grid2, kThreads, 0, st>>>(
            g->row_ptr, g->src_ptr, g->src_perm, geom, s.gstride, g->n_dst, g->n_src, x, s.C, wpk, s.n_rbf, A);
        return;
      }
    }
    const int nch = (s.C + kWave - 1) / kWave;
    const unsigned grid = ceil_div(static_cast<int64_t>(g->n_src) * 2 * nch, kWavesPerBlock);
    // one launch per degree part (each writes its own degrees' rows of A)
    auto go = [&](auto nrbf) {
      constexpr int NR = decltype(nrbf)::value;
      for_parts<InParts<LMAX, NR>>([&](auto lo, auto hi) {
        scatter_in_kernel<LMAX, MMAX, NR, T, TA, decltype(lo)::value, decltype(hi)::value><<<grid, kThreads, 0, st>>>(
            g->row_ptr, g->src_ptr, g->src_perm, geom, s.gstride, g->n_dst, g->n_src, x, s.C, wrad, s.n_rbf, A);
      });
    };
    if (s.n_rbf <= 8)
      go(std::integral_constant<int, 8>{});
    else
      go(std::integral_constant<int, 16>{});
  }
  template <typename T>
  static void aggregate(const egnn_graph *g, const LayerShape &s, const float *geom, const Acts &a, const T *x,
                        T *x_out, T *edge_out, hipStream_t st) {
    CPtr3 Y{{a.Y[0], a.Y[1], a.Y[2]}};
    if constexpr (std::is_same<T, uint16_t>::value && LMAX <= 6) {  // (at degree 8 the pair kernel spills)
      if (s.C % (2 * kWave) == 0) {  // channel pairs
        const unsigned grid2 = ceil_div(static_cast<int64_t>(g->n_dst) * (s.C / (2 * kWave)), kWavesPerBlock);
        aggregate_pair_kernel<LMAX, MMAX><<<grid2, kThreads, 0, st>>>(g->row_ptr, g->n_dst, geom, s.gstride, a.alpha,
                                                                      Y, s.C, x, x_out, edge_out);
        return;
      }
    }
    const int nch = (s.C + kWave - 1) / kWave;
    const unsigned grid = ceil_div(static_cast<int64_t>(g->n_dst) * nch, kWavesPerBlock);
    // one launch per degree part (each writes its own coefficients of x_out and edge_out)
    for_parts<AggParts<LMAX>>([&](auto lo, auto hi) {
      aggregate_kernel<LMAX, MMAX, T, decltype(lo)::value, decltype(hi)::value><<<grid, kThreads, 0, st>>>(
          g->row_ptr, g->n_dst, geom, s.gstride, s.nD + s.n_rbf, a.alpha, Y, s.C, x, x_out, edge_out);
    });
  }
  template <typename TY>
  static void bwd_row_t(const egnn_graph *g, const LayerShape &s, const float *geom, const Acts &a, const float *G,
                        const float *w_att, const BwdWs &w, hipStream_t st) {
    CPtr3 Y{{a.Y[0], a.Y[1], a.Y[2]}};
    constexpr bool bf = std::is_same<TY, uint16_t>::value;
    Ptr3 dY = bf ? Ptr3{{w.dYb[0], w.dYb[1], w.dYb[2]}} : Ptr3{{w.dY[0], w.dY[1], w.dY[2]}};
    const unsigned grid = ceil_div(g->n_dst, kWavesPerBlock);
    if (bf && s.C == 2 * kWave)
      bwd_row_pair_kernel<LMAX, MMAX><<<grid, kThreads, 0, st>>>(g->row_ptr, g->n_dst, geom, s.gstride, a.alpha, Y, s.C,
                                                                 G, w_att, dY, w.dalpha, w.watt_part);
    else if constexpr (LMAX >= 6) {  // degree parts: every dot first, then each part's dY
      auto go = [&](auto cpl) {
        constexpr int CP = decltype(cpl)::value;
        for_parts<RowParts<LMAX>>([&](auto lo, auto hi) {
          bwd_row_dot_kernel<LMAX, MMAX, CP, TY, decltype(lo)::value, decltype(hi)::value>
              <<<grid, kThreads, 0, st>>>(g->row_ptr, g->n_dst, geom, s.gstride, Y, s.C, G, w.dalpha);
        });
        for_parts<RowParts<LMAX>>([&](auto lo, auto hi) {
          bwd_row_grad_kernel<LMAX, MMAX, CP, TY, TY, decltype(lo)::value, decltype(hi)::value><<<grid, kThreads, 0, st>>>(
              g->row_ptr, g->n_dst, geom, s.gstride, a.alpha, Y, s.C, G, w_att, dY, w.dalpha, w.watt_part);
        });
      };
      if (s.C <= 64)
        go(std::integral_constant<int, 1>{});
      else  // C <= 128: egnn_layer_bwd rejects wider layers before any launch
        go(std::integral_constant<int, 2>{});
    } else if (s.C <= 64)
      bwd_row_kernel<LMAX, MMAX, 1, TY, TY><<<grid, kThreads, 0, st>>>(
          g->row_ptr, g->n_dst, geom, s.gstride, a.alpha, Y, s.C, G, w_att, dY, w.dalpha, w.watt_part);
    else  // C <= 128: egnn_layer_bwd rejects wider layers before any launch
      bwd_row_kernel<LMAX, MMAX, 2, TY, TY><<<grid, kThreads, 0, st>>>(
          g->row_ptr, g->n_dst, geom, s.gstride, a.alpha, Y, s.C, G, w_att, dY, w.dalpha, w.watt_part);
  }
  // dY is written in the storage type (bf16 feeds the bf16 GEMMs directly)
  static void bwd_row(const egnn_graph *g, const LayerShape &s, const float *geom, const Acts &a, const float *G,
                      const float *w_att, const BwdWs &w, hipStream_t st) {
    if (s.storage == EGNN_BF16)
      bwd_row_t<uint16_t>(g, s, geom, a, G, w_att, w, st);
    else
      bwd_row_t<float>(g, s, geom, a, G, w_att, w, st);
  }
  template <typename T>
  static void bwd_gate_t(const egnn_graph *g, const LayerShape &s, const float *geom, const T *x, const BwdWs &w,
                         hipStream_t st) {
    constexpr bool bf = std::is_same<T, uint16_t>::value;
    CPtr3 dA = bf ? CPtr3{{w.dAb[0], w.dAb[1], w.dAb[2]}} : CPtr3{{w.dA[0], w.dA[1], w.dA[2]}};
    const int nch = (s.C + kWave - 1) / kWave;
    const int ns = wrad_streams(g->n_src);
    const unsigned grid = ceil_div(static_cast<int64_t>(ns) * 2 * nch, kWavesPerBlock);
    // one launch per degree part (each writes its own gate pairs' partials)
    auto go = [&](auto nrbf) {
      constexpr int NR = decltype(nrbf)::value;
      for_parts<Parts<LMAX, NR>>([&](auto lo, auto hi) {
        wrad_grad_kernel<LMAX, MMAX, NR, T, decltype(lo)::value, decltype(hi)::value><<<grid, kThreads, 0, st>>>(
            g->row_ptr, g->src_ptr, g->src_perm, geom, s.gstride, g->n_dst, g->n_src, x, s.C, s.n_rbf, dA, ns,
            w.wrad_part);
      });
    };
    if (s.n_rbf <= 8)
      go(std::integral_constant<int, 8>{});
    else
      go(std::integral_constant<int, 16>{});
  }
  static void bwd_gate(const egnn_graph *g, const LayerShape &s, const float *geom, const void *x, const float *wrad,
                       const BwdWs &w, hipStream_t st) {
    (void)wrad;
    if (s.storage == EGNN_BF16)
      bwd_gate_t<uint16_t>(g, s, geom, static_cast<const uint16_t *>(x), w, st);
    else
      bwd_gate_t<float>(g, s, geom, static_cast<const float *>(x), w, st);
  }
  // bf16 storage: the gates from wpk, the radial weights packed as bf16 pairs
  // (as every bf16 forward forms them); fp32: from wrad
  template <typename TdA>
  static void bwd_node_t(const egnn_graph *g, const LayerShape &s, const float *geom, const float *G,
                         const float *wrad, const uint32_t *wpk, CPtr3 dA, float *gx, hipStream_t st) {
    const int nch = (s.C + kWave - 1) / kWave;
    const unsigned grid = ceil_div(static_cast<int64_t>(g->n_src) * 2 * nch, kWavesPerBlock);
    // one launch per degree part (each writes its own coefficient rows of gx)
    auto go = [&](auto nrbf, auto pk) {
      constexpr int NR = decltype(nrbf)::value;
      constexpr bool P = decltype(pk)::value;
      for_parts<Parts<LMAX, NR>>([&](auto lo, auto hi) {
        gather_grad_kernel<LMAX, MMAX, NR, TdA, P, decltype(lo)::value, decltype(hi)::value>
            <<<grid, kThreads, 0, st>>>(g->row_ptr, g->src_ptr, g->src_perm, geom, s.gstride, g->n_dst, g->n_src, s.C,
                                        wrad, P ? wpk : nullptr, s.n_rbf, dA, G, gx);
      });
    };
    if constexpr (std::is_same<TdA, uint16_t>::value) {
      if (s.n_rbf <= 8)
        go(std::integral_constant<int, 8>{}, std::true_type{});
      else
        go(std::integral_constant<int, 16>{}, std::true_type{});
    } else {
      if (s.n_rbf <= 8)
        go(std::integral_constant<int, 8>{}, std::false_type{});
      else
        go(std::integral_constant<int, 16>{}, std::false_type{});
    }
  }
  static void bwd_node(const egnn_graph *g, const LayerShape &s, const float *geom, const float *G, const float *wrad,
                       const BwdWs &w, float *gx, hipStream_t st) {
    if (s.storage == EGNN_BF16)
      bwd_node_t<uint16_t>(g, s, geom, G, wrad, w.wpk, CPtr3{{w.dAb[0], w.dAb[1], w.dAb[2]}}, gx, st);
    else
      bwd_node_t<float>(g, s, geom, G, wrad, nullptr, CPtr3{{w.dA[0], w.dA[1], w.dA[2]}}, gx, st);
  }
};

template <int LMAX, int MMAX, typename T, typename TA>
void launch_rotate_in(const egnn_graph *g, const LayerShape &s, const float *geom, const void *x, const float *wrad,
                      const uint32_t *wpk, const Acts &a, hipStream_t st) {
  Launch<LMAX, MMAX>::template rotate_in<T, TA>(g, s, geom, static_cast<const T *>(x), wrad, wpk, a, st);
}
template <int LMAX, int MMAX>
void rotate_in_f32(const egnn_graph *g, const LayerShape &s, const float *geom, const void *x, const float *wrad,
                   const uint32_t *wpk, const Acts &a, hipStream_t st) {
  launch_rotate_in<LMAX, MMAX, float, float>(g, s, geom, x, wrad, wpk, a, st);
}
template <int LMAX, int MMAX>
void rotate_in_bf16(const egnn_graph *g, const LayerShape &s, const float *geom, const void *x, const float *wrad,
                    const uint32_t *wpk, const Acts &a, hipStream_t st) {
  launch_rotate_in<LMAX, MMAX, uint16_t, uint16_t>(g, s, geom, x, wrad, wpk, a, st);
}
template <int LMAX, int MMAX>
void aggregate_f32(const egnn_graph *g, const LayerShape &s, const float *geom, const Acts &a, const void *x,
                   void *x_out, void *edge_out, hipStream_t st) {
  Launch<LMAX, MMAX>::template aggregate<float>(g, s, geom, a, static_cast<const float *>(x),
                                                static_cast<float *>(x_out), static_cast<float *>(edge_out), st);
}
template <int LMAX, int MMAX>
void aggregate_bf16(const egnn_graph *g, const LayerShape &s, const float *geom, const Acts &a, const void *x,
                    void *x_out, void *edge_out, hipStream_t st) {
  Launch<LMAX, MMAX>::template aggregate<uint16_t>(g, s, geom, a, static_cast<const uint16_t *>(x),
                                                   static_cast<uint16_t *>(x_out), static_cast<uint16_t *>(edge_out),
                                                   st);
}
template <int LMAX, int MMAX>
void bwd_row_launch(const egnn_graph *g, const LayerShape &s, const float *geom, const Acts &a, const float *G,
                    const float *w_att, const BwdWs &w, hipStream_t st) {
  Launch<LMAX, MMAX>::bwd_row(g, s, geom, a, G, w_att, w, st);
}
template <int LMAX, int MMAX>
void bwd_gate_launch(const egnn_graph *g, const LayerShape &s, const float *geom, const void *x, const float *wrad,
                     const BwdWs &w, hipStream_t st) {
  Launch<LMAX, MMAX>::bwd_gate(g, s, geom, x, wrad, w, st);
}
template <int LMAX, int MMAX>
void bwd_node_launch(const egnn_graph *g, const LayerShape &s, const float *geom, const float *G, const float *wrad,
                     const BwdWs &w, float *gx, hipStream_t st) {
  Launch<LMAX, MMAX>::bwd_node(g, s, geom, G, wrad, w, gx, st);
}

template <int LMAX, int MMAX>
void edge_update_launch(int64_t E, const LayerShape &s, const float *geom, const Acts &a, const void *e_in, void *e_out,
                        hipStream_t st) {
  CPtr3 Y{{a.Y[0], a.Y[1], a.Y[2]}};
  int64_t blocks = (E + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 8192) blocks = 8192;
  const unsigned grid = static_cast<unsigned>(blocks);
  auto go = [&](auto cpl) {
    constexpr int CPL = decltype(cpl)::value;
    if (s.storage == EGNN_BF16)
      edge_update_kernel<LMAX, MMAX, CPL, uint16_t><<<grid, kThreads, 0, st>>>(
          E, geom, s.gstride, Y, s.C, static_cast<const uint16_t *>(e_in), static_cast<uint16_t *>(e_out));
    else
      edge_update_kernel<LMAX, MMAX, CPL, float><<<grid, kThreads, 0, st>>>(
          E, geom, s.gstride, Y, s.C, static_cast<const float *>(e_in), static_cast<float *>(e_out));
  };
  if (s.C <= kWave)
    go(std::integral_constant<int, 1>{});
  else if (s.C <= 2 * kWave)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, 4>{});
}
template <int LMAX, int MMAX>
void edge_dy_launch(int64_t E, const LayerShape &s, const float *geom, const float *dE, const BwdWs &w,
                    hipStream_t st) {
  int64_t blocks = (E + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 8192) blocks = 8192;
  const unsigned grid = static_cast<unsigned>(blocks);
  const bool bf = s.storage == EGNN_BF16;
  Ptr3 dY = bf ? Ptr3{{w.dYb[0], w.dYb[1], w.dYb[2]}} : Ptr3{{w.dY[0], w.dY[1], w.dY[2]}};
  auto go = [&](auto cpl) {
    constexpr int CPL = decltype(cpl)::value;
    if (bf)
      edge_dy_kernel<LMAX, MMAX, CPL, uint16_t><<<grid, kThreads, 0, st>>>(E, geom, s.gstride, dE, s.C, dY);
    else
      edge_dy_kernel<LMAX, MMAX, CPL, float><<<grid, kThreads, 0, st>>>(E, geom, s.gstride, dE, s.C, dY);
  };
  // C <= 128: the backward rejects wider layers before any launch
  if (s.C <= kWave)
    go(std::integral_constant<int, 1>{});
  else
    go(std::integral_constant<int, 2>{});
}

egnn_status check_graph(const egnn_graph *g) {
  EGNN_REQUIRE(g, "graph is null");
  EGNN_REQUIRE(g->n_dst >= 0 && g->n_src >= g->n_dst, "graph sizes invalid");
  EGNN_REQUIRE(g->n_edges >= 0 && g->n_edges <= g->capacity, "graph n_edges out of range");
  EGNN_REQUIRE(g->n_edges < (int64_t(1) << 31), "more than 2^31 edges");
  EGNN_REQUIRE(g->row_ptr, "row_ptr is null");
  if (g->n_edges > 0) EGNN_REQUIRE(g->src && g->src_ptr && g->src_perm, "graph arrays are null");
  return EGNN_OK;
}

}  // namespace
}  // namespace egnn

using namespace egnn;

extern "C" egnn_status egnn_layer_sizes(const egnn_layer_desc *d, const egnn_graph *g, size_t *saved_bytes,
                                        size_t *ws_fwd_bytes, size_t *ws_bwd_bytes) {
  clear_error();
  LayerShape s;
  EGNN_REQUIRE(make_shape(d, &s), "invalid layer description");
  egnn_status st = check_graph(g);
  if (st != EGNN_OK) return st;
  const int64_t E = g->n_edges;
  if (saved_bytes) {
    Carver cv{nullptr};
    carve_acts(cv, s, E);
    *saved_bytes = cv.off;
  }
  if (ws_fwd_bytes) {
    Carver cv{nullptr};
    carve_fwd_ws(cv, s, E);
    carve_acts(cv, s, E);  // used when no saved buffer is given
    *ws_fwd_bytes = cv.off;
  }
  if (ws_bwd_bytes) {
    Carver cv{nullptr};
    carve_bwd_ws(cv, s, E, g->n_dst, g->n_src);
    *ws_bwd_bytes = cv.off;
  }
  return EGNN_OK;
}

// The node block (attention + aggregation onto the destination) and the edge
// block (the per-edge message added to the edge embedding) share every step up
// to the SO(2) products.
static egnn_status layer_fwd_impl(bool edge_block, const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                  const float *weights, const void *x_in, void *x_out, void *edge_out,
                                  const void *e_in, void *e_out, void *saved, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  clear_error();
  LayerShape s;
  EGNN_REQUIRE(make_shape(d, &s), "invalid layer description");
  egnn_status st = check_graph(g);
  if (st != EGNN_OK) return st;
  EGNN_REQUIRE(weights && x_in, "null pointer");
  if (edge_block) {
    EGNN_REQUIRE(g->n_edges == 0 || (e_in && e_out), "edge embeddings are null");
  } else {
    EGNN_REQUIRE(x_out, "null pointer");
    EGNN_REQUIRE(x_in != x_out, "x_out must not alias x_in");
  }
  EGNN_REQUIRE(aligned16(ws) && aligned16(saved), "ws and saved must be 16-byte aligned");
  const int64_t E = g->n_edges;
  if (E > 0) EGNN_REQUIRE(geom, "geom is null");
  Carver cw{static_cast<char *>(ws)};
  FwdWs fw = carve_fwd_ws(cw, s, E);
  Acts acts;
  if (saved) {
    Carver cs{static_cast<char *>(saved)};
    acts = carve_acts(cs, s, E);
  } else {
    acts = carve_acts(cw, s, E);
  }
  if (!ws || ws_bytes < cw.off) {
    set_error("workspace of %zu bytes, need %zu", ws_bytes, cw.off);
    return EGNN_E_WORKSPACE;
  }
  const WOff wo = weight_offsets(s);
  const bool bf = s.storage == EGNN_BF16;
  const int T = 256;
  // expanded weights
  for (int m = 0; m <= s.mmax; ++m) {
    if (m == 0) {
      if (bf) {
        const int64_t n = static_cast<int64_t>(s.Ng[0]) * s.Kg[0];
        to_bf16_kernel<<<ceil_div(n, T), T, 0, stream>>>(weights + wo.W0, n, static_cast<uint16_t *>(fw.B[0]));
      }
      continue;
    }
    const int rows = s.Ng[m] / 2, cols = s.Kg[m] / 2;
    const int64_t n = static_cast<int64_t>(4) * rows * cols;
    if (bf) {
      expand_weights_kernel<uint16_t><<<ceil_div(n, T), T, 0, stream>>>(weights + wo.W1[m], weights + wo.W2[m], rows,
                                                                      cols, static_cast<uint16_t *>(fw.B[m]));
    } else {
      // V+ = W1, V- = W2: V2 = W2 - W1, V3 = W1 + W2
      const int64_t nb = static_cast<int64_t>(rows) * cols;
      float *v = static_cast<float *>(fw.B[m]);
      combo_weights_kernel<<<ceil_div(nb, T), T, 0, stream>>>(weights + wo.W1[m], weights + wo.W2[m], nb, -1.f, 1.f,
                                                              1.f, 1.f, v, v + nb);
    }
  }
  if (bf) {
    const int64_t n = static_cast<int64_t>(8) * s.n_pairs * 2 * s.C;
    pack_wrad_kernel<<<ceil_div(n, T), T, 0, stream>>>(weights + wo.wrad, s.n_rbf, s.n_pairs, 2 * s.C, fw.wpk);
  }
  const double xb = bf ? 2.0 : 4.0;
  double sumK = 0, sumN = 0;
  for (int m = 0; m <= s.mmax; ++m) {
    sumK += s.Kg[m];
    sumN += s.Ng[m];
  }
  if (E > 0) {
    {
      const double bytes = double(g->n_src) * s.K * s.C * xb + double(E) * (s.nD + s.n_rbf + 1) * 4.0 +
                           double(E) * 4.0 + double(E) * sumK * xb;
      Timed t(stream, "rotate_in", 0.0, bytes);
      if (bf) {
        EGNN_DISPATCH_LM(s.lmax, s.mmax, rotate_in_bf16, g, s, geom, x_in, weights + wo.wrad, fw.wpk, acts, stream);
      } else {
        EGNN_DISPATCH_LM(s.lmax, s.mmax, rotate_in_f32, g, s, geom, x_in, weights + wo.wrad, nullptr, acts, stream);
      }
    }
    for (int m = 0; m <= s.mmax; ++m) {
      hipError_t e;
      if (!bf && m > 0) {
        // complex product, three real products (executed FLOPs = 3/4 of the four-product count)
        const int Np = s.Ng[m] / 2, Kp = s.Kg[m] / 2;
        const float *A = static_cast<const float *>(acts.A[m]);
        const float *v = static_cast<const float *>(fw.B[m]);
        const int64_t nb = static_cast<int64_t>(Np) * Kp;
        Timed t(stream, "cgemm_fwd_f32", 2.0 * double(E) * s.Ng[m] * s.Kg[m], double(E) * (s.Kg[m] * xb + s.Ng[m] * 4.0));
        e = cgemm_f32(static_cast<int>(E), Np, Kp, A, A + Kp, s.Kg[m], true, weights + wo.W1[m], v, v + nb, Kp, true,
                      1.0f, static_cast<float *>(acts.Y[m]), static_cast<float *>(acts.Y[m]) + Np, s.Ng[m], 1, 0,
                      stream);
        if (e != hipSuccess) {
          set_error("GEMM launch failed: %s", hipGetErrorString(e));
          return EGNN_E_HIP;
        }
        continue;
      }
      Timed t(stream, bf ? "gemm_nt_bf16" : "gemm_nt_f32", 2.0 * double(E) * s.Ng[m] * s.Kg[m],
              double(E) * (s.Kg[m] + s.Ng[m]) * xb);
      if (bf) {
        e = gemm_bf16_nt(static_cast<int>(E), s.Ng[m], s.Kg[m], static_cast<const uint16_t *>(acts.A[m]), s.Kg[m],
                         static_cast<const uint16_t *>(fw.B[m]), s.Kg[m], acts.Y[m], s.Ng[m], true, stream);
      } else {
        const float *B = m == 0 ? weights + wo.W0 : static_cast<const float *>(fw.B[m]);
        e = gemm_f32(static_cast<int>(E), s.Ng[m], s.Kg[m], static_cast<const float *>(acts.A[m]), s.Kg[m], true, B,
                     s.Kg[m], true, static_cast<float *>(acts.Y[m]), s.Ng[m], 1, 0, stream);
      }
      if (e != hipSuccess) {
        set_error("GEMM launch failed: %s", hipGetErrorString(e));
        return e == hipErrorNotSupported ? EGNN_E_UNSUPPORTED : EGNN_E_HIP;
      }
    }
  }
  if (edge_block) {
    if (E > 0) {
      // Y read, e read and written, D rows
      Timed t(stream, "edge_update", 0.0, double(E) * (sumN * xb + 2.0 * s.K * s.C * xb + s.nD * 4.0));
      EGNN_DISPATCH_LM(s.lmax, s.mmax, edge_update_launch, E, s, geom, acts, e_in, e_out, stream);
    }
  } else if (g->n_dst > 0) {
    if (E > 0) {
      Timed t(stream, "attention", 0.0, double(E) * (s.C * 4.0 + 8.0));
      if (bf)
        attention_kernel<uint16_t><<<ceil_div(g->n_dst, kWavesPerBlock), kThreads, 0, stream>>>(
            g->row_ptr, g->n_dst, static_cast<const uint16_t *>(acts.Y[0]), s.Ng[0], s.C, weights + wo.watt, fw.logit,
            acts.alpha);
      else
        attention_kernel<float><<<ceil_div(g->n_dst, kWavesPerBlock), kThreads, 0, stream>>>(
            g->row_ptr, g->n_dst, static_cast<const float *>(acts.Y[0]), s.Ng[0], s.C, weights + wo.watt, fw.logit,
            acts.alpha);
    }
    const double bytes = double(E) * (sumN * xb + s.nD * 4.0 + 4.0) + 2.0 * g->n_dst * s.K * s.C * xb +
                         (edge_out ? double(E) * s.K * s.C * xb : 0.0);
    Timed t(stream, "aggregate", 0.0, bytes);
    if (bf) {
      EGNN_DISPATCH_LM(s.lmax, s.mmax, aggregate_bf16, g, s, geom, acts, x_in, x_out, edge_out, stream);
    } else {
      EGNN_DISPATCH_LM(s.lmax, s.mmax, aggregate_f32, g, s, geom, acts, x_in, x_out, edge_out, stream);
    }
  }
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}

extern "C" egnn_status egnn_layer_fwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                      const float *weights, const void *x_in, void *x_out, void *edge_out,
                                      void *saved, void *ws, size_t ws_bytes, hipStream_t stream) {
  return layer_fwd_impl(false, d, g, geom, weights, x_in, x_out, edge_out, nullptr, nullptr, saved, ws, ws_bytes,
                        stream);
}

extern "C" egnn_status egnn_edge_update_fwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                            const float *weights, const void *x_in, const void *e_in, void *e_out,
                                            void *saved, void *ws, size_t ws_bytes, hipStream_t stream) {
  return layer_fwd_impl(true, d, g, geom, weights, x_in, nullptr, nullptr, e_in, e_out, saved, ws, ws_bytes, stream);
}

// Node block: grad_out = dL/dx' [n_dst][K][C].  Edge block: grad_out =
// dL/de' [n_edges][K][C]; its first step is dY = trunc(D dE) in place of the
// attention-weighted row kernel, there is no w_att gradient and no node
// residual.
static egnn_status layer_bwd_impl(bool edge_block, const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                  const float *weights, const void *x_in, const void *saved, const float *grad_out,
                                  float *grad_x_in, float *grad_weights, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  clear_error();
  LayerShape s;
  EGNN_REQUIRE(make_shape(d, &s), "invalid layer description");
  egnn_status st = check_graph(g);
  if (st != EGNN_OK) return st;
  if (s.C > 128) {
    set_error("the backward pass supports C <= 128");
    return EGNN_E_UNSUPPORTED;
  }
  EGNN_REQUIRE(weights && x_in && saved && grad_x_in && grad_weights, "null pointer");
  EGNN_REQUIRE((edge_block ? g->n_edges : g->n_dst) == 0 || grad_out, "grad_out is null");
  EGNN_REQUIRE(aligned16(ws) && aligned16(saved), "ws and saved must be 16-byte aligned");
  const int64_t E = g->n_edges;
  if (E > 0) EGNN_REQUIRE(geom, "geom is null");
  Carver cs{static_cast<char *>(const_cast<void *>(saved))};
  const Acts acts = carve_acts(cs, s, E);
  Carver cw{static_cast<char *>(ws)};
  const BwdWs w = carve_bwd_ws(cw, s, E, g->n_dst, g->n_src);
  if (!ws || ws_bytes < cw.off) {
    set_error("workspace of %zu bytes, need %zu", ws_bytes, cw.off);
    return EGNN_E_WORKSPACE;
  }
  const WOff wo = weight_offsets(s);
  const int T = 256;
  const bool bf = s.storage == EGNN_BF16;
  fill_f32<<<ceil_div(wo.total, T), T, 0, stream>>>(grad_weights, wo.total, 0.0f);
  for (int m = 0; m <= s.mmax; ++m) {
    if (bf) {
      // bf16: B_m^T (expanded for m >= 1) for dA_m = dY_m B_m
      const int64_t n = static_cast<int64_t>(s.Ng[m]) * s.Kg[m];
      if (m == 0)
        expand_weights_t_kernel<<<ceil_div(n, T), T, 0, stream>>>(weights + wo.W0, nullptr, s.Ng[0], s.Kg[0], false,
                                                                  w.BT[0]);
      else
        expand_weights_t_kernel<<<ceil_div(n, T), T, 0, stream>>>(weights + wo.W1[m], weights + wo.W2[m],
                                                                  s.Ng[m] / 2, s.Kg[m] / 2, true, w.BT[m]);
    } else if (m > 0) {
      // input gradient multiplies by conj(W): V+ = W1, V- = -W2, so V2 = -W1 - W2, V3 = W1 - W2
      const int64_t nb = static_cast<int64_t>(s.Ng[m] / 2) * (s.Kg[m] / 2);
      combo_weights_kernel<<<ceil_div(nb, T), T, 0, stream>>>(weights + wo.W1[m], weights + wo.W2[m], nb, -1.f, -1.f,
                                                              1.f, -1.f, w.B[m], w.B[m] + nb);
    }
  }
  double sumK = 0, sumN = 0;
  for (int m = 0; m <= s.mmax; ++m) {
    sumK += s.Kg[m];
    sumN += s.Ng[m];
  }
  if (edge_block && E > 0) {
    // dE read, dY written (storage type), D rows
    Timed t(stream, "edge_dy", 0.0, double(E) * (s.K * s.C * 4.0 + sumN * (bf ? 2.0 : 4.0) + s.nD * 4.0));
    EGNN_DISPATCH_LM(s.lmax, s.mmax, edge_dy_launch, E, s, geom, grad_out, w, stream);
  }
  if (!edge_block && g->n_dst > 0 && E > 0) {
    {
      // G rows, Y read and dY written (storage type), D rows, alpha / dalpha, w_att partials
      const double yb = bf ? 2.0 : 4.0;
      const double bytes = double(g->n_dst) * s.K * s.C * 4.0 + double(E) * (2.0 * sumN * yb + s.nD * 4.0 + 12.0) +
                           double(g->n_dst) * s.C * 4.0;
      Timed t(stream, "bwd_row", 0.0, bytes);
      EGNN_DISPATCH_LM(s.lmax, s.mmax, bwd_row_launch, g, s, geom, acts, grad_out, weights + wo.watt, w, stream);
    }
    // w_att gradient: fixed-order sum of the per-row partials (the split-K
    // partial buffer is free until the weight-gradient products below)
    colsum_fixed(w.watt_part, g->n_dst, s.C, s.C, grad_weights + wo.watt, w.P, w.P_floats, stream);
  }
  if (E > 0 && bf) {
    // bf16 storage: both gradient products on bf16 MFMA, fp32 accumulate.
    //   dA_m = dY_m B_m                 (dY in bf16 from bwd_row, B_m^T prepared above)
    //   dB_m = sum_e dY_m[e]^T A_m[e]   (both read as stored, edges as rows; split
    //                                    over edges, summed in order)
    // then dW_m1, dW_m2 folded out of dB_m for m >= 1.
    for (int m = 0; m <= s.mmax; ++m) {
      const int Ng = s.Ng[m], Kg = s.Kg[m];
      hipError_t e;
      {
        Timed t(stream, "gemm_dx_bf16", 2.0 * double(E) * Ng * Kg, double(E) * (Ng + Kg) * 2.0);
        e = gemm_bf16_nt(static_cast<int>(E), Kg, Ng, w.dYb[m], Ng, w.BT[m], Ng, w.dAb[m], Kg, true, stream);
      }
      if (e != hipSuccess) {
        set_error("GEMM launch failed: %s", hipGetErrorString(e));
        return EGNN_E_HIP;
      }
      const int64_t pn = static_cast<int64_t>(Ng) * Kg;
      const int splits =
          dw_splits_for(E, gemm_bf16_tn_tiles(Ng, Kg), pn, w.P_floats, gemm_bf16_tn_blocks_per_cu(), xcd_cus());
      {
        Timed t(stream, "gemm_dw_bf16", 2.0 * double(E) * Ng * Kg, double(E) * (Ng + Kg) * 2.0 + double(splits) * pn * 4.0);
        e = gemm_bf16_tn_splitk(Ng, Kg, static_cast<int>(E), w.dYb[m], Ng, static_cast<const uint16_t *>(acts.A[m]), Kg,
                                w.P, Kg, splits, pn, stream);
      }
      if (e != hipSuccess) {
        set_error("GEMM launch failed: %s", hipGetErrorString(e));
        return EGNN_E_HIP;
      }
      if (m == 0) {
        colsum(w.P, splits, pn, pn, grad_weights + wo.W0, stream);
      } else {
        colsum(w.P, splits, pn, pn, w.dWexp, stream);
        const int64_t nb = pn / 4;
        fold_expanded_kernel<<<ceil_div(nb, T), T, 0, stream>>>(w.dWexp, Ng / 2, Kg / 2, grad_weights + wo.W1[m],
                                                                grad_weights + wo.W2[m]);
      }
    }
  } else if (E > 0) {
    for (int m = 0; m <= s.mmax; ++m) {
      hipError_t e;
      if (m > 0) {
        const int Np = s.Ng[m] / 2, Kp = s.Kg[m] / 2;
        const int64_t nb = static_cast<int64_t>(Np) * Kp;
        const float *A = static_cast<const float *>(acts.A[m]);
        {
          // (dX+ + i dX-) = sum_n (dY+ + i dY-)(n) conj(W)(n, k)
          Timed t(stream, "cgemm_dx_f32", 2.0 * double(E) * s.Ng[m] * s.Kg[m], double(E) * (s.Ng[m] + s.Kg[m]) * 4.0);
          e = cgemm_f32(static_cast<int>(E), Kp, Np, w.dY[m], w.dY[m] + Np, s.Ng[m], true, weights + wo.W1[m], w.B[m],
                        w.B[m] + nb, Kp, false, 1.0f, w.dA[m], w.dA[m] + Kp, s.Kg[m], 1, 0, stream);
        }
        if (e != hipSuccess) {
          set_error("GEMM launch failed: %s", hipGetErrorString(e));
          return EGNN_E_HIP;
        }
        const int splits = dw_splits_for(E, gemm_f32_tiles(Np, Kp), 2 * nb, w.P_floats,
                                         cgemm_f32_dw_blocks_per_cu(Np, Kp), xcd_cus());
        {
          // dW1 + i dW2 = sum_e (dY+ + i dY-)^T (X+ - i X-), split over edges
          Timed t(stream, "cgemm_dw_f32", 2.0 * double(E) * s.Ng[m] * s.Kg[m],
                  double(E) * (s.Ng[m] + s.Kg[m]) * 4.0 + 2.0 * double(splits) * nb * 4.0);
          e = cgemm_f32(Np, Kp, static_cast<int>(E), w.dY[m], w.dY[m] + Np, s.Ng[m], false, A, A + Kp, nullptr,
                        s.Kg[m], false, -1.0f, w.P, w.P + splits * nb, Kp, splits, nb, stream);
        }
        if (e != hipSuccess) {
          set_error("GEMM launch failed: %s", hipGetErrorString(e));
          return EGNN_E_HIP;
        }
        colsum(w.P, splits, nb, nb, grad_weights + wo.W1[m], stream);
        colsum(w.P + splits * nb, splits, nb, nb, grad_weights + wo.W2[m], stream);
        continue;
      }
      const float *B = weights + wo.W0;
      // dA_0 = dY_0 W0
      {
        Timed t(stream, "gemm_nn_f32", 2.0 * double(E) * s.Ng[m] * s.Kg[m], double(E) * (s.Ng[m] + s.Kg[m]) * 4.0);
        e = gemm_f32(static_cast<int>(E), s.Kg[m], s.Ng[m], w.dY[m], s.Ng[m], true, B, s.Kg[m], false,
                              w.dA[m], s.Kg[m], 1, 0, stream);
      }
      if (e != hipSuccess) {
        set_error("GEMM launch failed: %s", hipGetErrorString(e));
        return EGNN_E_HIP;
      }
      // dB_m = dY_m^T A_m, split over edges, then summed in order
      const int64_t pn = static_cast<int64_t>(s.Ng[m]) * s.Kg[m];
      const int splits = dw_splits_for(E, gemm_f32_tiles(s.Ng[m], s.Kg[m]), pn, w.P_floats,
                                       gemm_f32_tn_blocks_per_cu(s.Ng[m], s.Kg[m]), xcd_cus());
      {
        Timed t(stream, "gemm_tn_f32", 2.0 * double(E) * s.Ng[m] * s.Kg[m],
                double(E) * (s.Ng[m] + s.Kg[m]) * 4.0 + double(splits) * pn * 4.0);
        e = gemm_f32(s.Ng[m], s.Kg[m], static_cast<int>(E), w.dY[m], s.Ng[m], false,
                     static_cast<const float *>(acts.A[m]), s.Kg[m], false, w.P, s.Kg[m], splits, pn, stream);
      }
      if (e != hipSuccess) {
        set_error("GEMM launch failed: %s", hipGetErrorString(e));
        return EGNN_E_HIP;
      }
      colsum(w.P, splits, pn, pn, grad_weights + wo.W0, stream);
    }
  }
  if (E > 0) {
    const int ncol = s.n_pairs * 2 * s.C;
    {
      // dA read once; the edge-frame input is recomputed from each node's own row
      const double xb = bf ? 2.0 : 4.0;
      const double bytes = double(g->n_src) * s.K * s.C * xb + double(E) * (s.nD + s.n_rbf + 1) * 4.0 + double(E) * 4.0 +
                           double(E) * sumK * xb;
      Timed t(stream, "bwd_gate", 0.0, bytes);
      EGNN_DISPATCH_LM(s.lmax, s.mmax, bwd_gate_launch, g, s, geom, x_in, weights + wo.wrad, w, stream);
    }
    const int64_t nw = static_cast<int64_t>(s.n_rbf) * ncol;
    const int ns = wrad_streams(g->n_src);
    // (the split-K partial buffer is free again: its sums are done)
    colsum_fixed(w.wrad_part, ns, nw, nw, grad_weights + wo.wrad, w.P, w.P_floats, stream);
  }
  if (g->n_src > 0) {
    if (E == 0) {
      // no edges: dx = G on owned rows, 0 on ghosts
      const int64_t n = static_cast<int64_t>(g->n_src) * s.K * s.C;
      fill_f32<<<ceil_div(n, T), T, 0, stream>>>(grad_x_in, n, 0.0f);
      if (g->n_dst > 0 && !edge_block)
        EGNN_TRY_HIP(hipMemcpyAsync(grad_x_in, grad_out, sizeof(float) * g->n_dst * s.K * s.C, hipMemcpyDeviceToDevice,
                                    stream));
    } else {
      const double bytes = double(E) * (sumK * (bf ? 2.0 : 4.0) + s.nD * 4.0 + 8.0) + double(g->n_dst) * s.K * s.C * 4.0 +
                           double(g->n_src) * s.K * s.C * 4.0;
      if (bf) {  // the gates of every bf16 forward: bf16 radial weights (8 basis pairs: up to 16 functions)
        const int64_t n = static_cast<int64_t>(8) * s.n_pairs * 2 * s.C;
        pack_wrad_kernel<<<ceil_div(n, T), T, 0, stream>>>(weights + wo.wrad, s.n_rbf, s.n_pairs, 2 * s.C, w.wpk);
      }
      Timed t(stream, "bwd_node", 0.0, bytes);
      EGNN_DISPATCH_LM(s.lmax, s.mmax, bwd_node_launch, g, s, geom, edge_block ? nullptr : grad_out,
                       weights + wo.wrad, w, grad_x_in, stream);
    }
  }
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}

extern "C" egnn_status egnn_layer_bwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                      const float *weights, const void *x_in, const void *saved,
                                      const float *grad_out, float *grad_x_in, float *grad_weights, void *ws,
                                      size_t ws_bytes, hipStream_t stream) {
  return layer_bwd_impl(false, d, g, geom, weights, x_in, saved, grad_out, grad_x_in, grad_weights, ws, ws_bytes,
                        stream);
}

extern "C" egnn_status egnn_edge_update_bwd(const egnn_layer_desc *d, const egnn_graph *g, const float *geom,
                                            const float *weights, const void *x_in, const void *saved,
                                            const float *grad_e_out, float *grad_x_in, float *grad_weights, void *ws,
                                            size_t ws_bytes, hipStream_t stream) {
  return layer_bwd_impl(true, d, g, geom, weights, x_in, saved, grad_e_out, grad_x_in, grad_weights, ws, ws_bytes,
                        stream);
}
