// Label -> Matrix: orbital Hamiltonian blocks from edge / node irreps.
//
// MALOQ Sec. III-B1, Eq. (1): the block between a shell of degree la and one
// of degree lb is la (x) lb, written through Clebsch-Gordan coefficients as
// the direct sum of degrees L = |la-lb|..la+lb; all |L,M> of a block form its
// label vector.  Sec. III-B2 describes a CUDA kernel with one thread per
// matrix element and one thread block per node or edge, driven by a
// precomputed orbital template.  Here one 64-lane wave owns a row (edge or
// node): the row's irreps are staged in LDS, lanes first form the labels
// h_L = W_L f^L (one label per lane), then lanes form the block entries from a
// precomputed sparse list of real CG terms per entry (the orbital template).
//
// The real couplings are built on the host (cg_real.h).
#include <cmath>
#include <complex>
#include <cstring>
#include <mutex>
#include <vector>

#include "cg_real.h"
#include "common.h"
#include "timing.h"

namespace egnn {
namespace {

constexpr int kSlots = 8;
constexpr int kMaxOrb = 32;
constexpr int kMaxEntries = kMaxOrb * kMaxOrb;
constexpr int kMaxTerms = 8192;
constexpr int kMaxLab = kMaxEntries;

constexpr int kMaxShellL = 4;          // shells up to g
constexpr int kMaxLabL = 2 * kMaxShellL;  // labels up to L = 8 (irreps lmax 8)
constexpr int kMaxNL = 64;             // label channels per degree (4 MFMA column tiles)

struct Table {
  int lmax_lab;                        // 2 * max shell degree
  int nL[kMaxLabL + 1];                // label channels per L
  int woff[kMaxLabL + 2];              // first weight row of L
  int hoff[kMaxLabL + 2];              // first label of L in the (L, M, k) order
  int term_start[kMaxEntries + 1];
  float term_coef[kMaxTerms];
  unsigned short term_idx[kMaxTerms];
  unsigned short lab_w[kMaxLab];   // weight row of label q
  unsigned short lab_f[kMaxLab];   // irreps coefficient index L^2 + L + M of label q
};

__device__ Table g_tables[kSlots];

using cg::real_coupling;

struct Layout {
  int n_orb = 0, n_w = 0, n_lab = 0;
  std::vector<int> nL, woff;  // label rows per L, first weight row of L
  Table t;
};

bool build_layout(const int *shell_l, int n_shells, Layout *out) {
  std::vector<int> off(n_shells);
  int o = 0, lmx = 0;
  for (int a = 0; a < n_shells; ++a) {
    if (shell_l[a] < 0 || shell_l[a] > kMaxShellL) return false;
    off[a] = o;
    o += 2 * shell_l[a] + 1;
    lmx = std::max(lmx, shell_l[a]);
  }
  if (o > kMaxOrb) return false;
  const int Lmax = 2 * lmx;
  out->n_orb = o;
  out->nL.assign(Lmax + 1, 0);
  struct Item { int a, b, L, k; };
  std::vector<Item> items;
  for (int a = 0; a < n_shells; ++a)
    for (int b = 0; b < n_shells; ++b)
      for (int L = std::abs(shell_l[a] - shell_l[b]); L <= shell_l[a] + shell_l[b]; ++L)
        items.push_back({a, b, L, out->nL[L]++});
  out->woff.assign(Lmax + 2, 0);
  for (int L = 0; L <= Lmax; ++L) out->woff[L + 1] = out->woff[L] + out->nL[L];
  out->n_w = out->woff[Lmax + 1];
  // label q enumerates (L, M, k): offset(L) + (M + L) * n_L + k
  std::vector<int> hoff(Lmax + 2, 0);
  for (int L = 0; L <= Lmax; ++L) hoff[L + 1] = hoff[L] + (2 * L + 1) * out->nL[L];
  out->n_lab = hoff[Lmax + 1];
  if (out->n_lab > kMaxLab || out->n_w > 65535) return false;
  for (int L = 0; L <= Lmax; ++L)
    if (out->nL[L] > kMaxNL) return false;
  Table &t = out->t;
  std::memset(&t, 0, sizeof(t));
  t.lmax_lab = Lmax;
  for (int L = 0; L <= Lmax; ++L) {
    t.nL[L] = out->nL[L];
    t.woff[L] = out->woff[L];
    t.hoff[L] = hoff[L];
  }
  t.woff[Lmax + 1] = out->woff[Lmax + 1];
  t.hoff[Lmax + 1] = hoff[Lmax + 1];
  for (int L = 0; L <= Lmax; ++L)
    for (int M = -L; M <= L; ++M)
      for (int k = 0; k < out->nL[L]; ++k) {
        const int q = hoff[L] + (M + L) * out->nL[L] + k;
        t.lab_w[q] = static_cast<unsigned short>(out->woff[L] + k);
        t.lab_f[q] = static_cast<unsigned short>(L * L + L + M);
      }
  // sparse terms per block entry
  std::vector<std::vector<std::pair<float, int>>> terms(static_cast<size_t>(o) * o);
  for (const Item &it : items) {
    const int la = shell_l[it.a], lb = shell_l[it.b];
    std::vector<double> Q = real_coupling(la, lb, it.L);
    const int nb = 2 * lb + 1, nLL = 2 * it.L + 1;
    for (int i = 0; i < 2 * la + 1; ++i)
      for (int j = 0; j < nb; ++j)
        for (int M = 0; M < nLL; ++M) {
          const double c = Q[(i * nb + j) * nLL + M];
          if (std::fabs(c) < 1e-12) continue;
          const int q = hoff[it.L] + M * out->nL[it.L] + it.k;
          terms[(off[it.a] + i) * o + (off[it.b] + j)].push_back({static_cast<float>(c), q});
        }
  }
  int n = 0;
  for (int r = 0; r < o * o; ++r) {
    t.term_start[r] = n;
    for (auto &p : terms[r]) {
      if (n >= kMaxTerms) return false;
      t.term_coef[n] = p.first;
      t.term_idx[n] = static_cast<unsigned short>(p.second);
      ++n;
    }
  }
  t.term_start[o * o] = n;
  return true;
}

struct SlotKey {
  int device;
  int n;
  int l[16];
};
struct SlotCache {
  std::mutex mu;
  SlotKey keys[64][kSlots];
  int used[64] = {0};
};
SlotCache g_cache;

// Slot of the table for (device, shell list); fills it on first use.
egnn_status table_slot(const int *shell_l, int n_shells, int *slot, Layout *lay) {
  int dev = 0;
  EGNN_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) {
    set_error("device index %d out of range", dev);
    return EGNN_E_UNSUPPORTED;
  }
  if (!build_layout(shell_l, n_shells, lay)) {
    set_error("shell list not supported (each l <= %d, at most %d orbitals)", kMaxShellL, kMaxOrb);
    return EGNN_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_cache.mu);
  for (int s = 0; s < g_cache.used[dev]; ++s) {
    const SlotKey &k = g_cache.keys[dev][s];
    if (k.n == n_shells && std::memcmp(k.l, shell_l, sizeof(int) * n_shells) == 0) {
      *slot = s;
      return EGNN_OK;
    }
  }
  if (g_cache.used[dev] >= kSlots) {
    set_error("more than %d distinct shell lists on one device", kSlots);
    return EGNN_E_UNSUPPORTED;
  }
  const int s = g_cache.used[dev];
  EGNN_TRY_HIP(hipMemcpyToSymbol(HIP_SYMBOL(g_tables), &lay->t, sizeof(Table), sizeof(Table) * s,
                                 hipMemcpyHostToDevice));
  SlotKey &k = g_cache.keys[dev][s];
  k.device = dev;
  k.n = n_shells;
  std::memcpy(k.l, shell_l, sizeof(int) * n_shells);
  g_cache.used[dev] = s + 1;
  *slot = s;
  return EGNN_OK;
}

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kTile = 16;  // rows per wave tile (the MFMA M dimension)
constexpr int kValuLabels = 2;  // label channels of one degree up to which the VALU forms them

// Labels by MFMA, entries from the LDS-resident template.  For each (L, M),
// the 16 rows x C channels of the tile times W_L^T (C x n_L) is a chain of
// v_mfma_f32_16x16x4f32 over S = C/4 channel steps.  Lane l feeds row l % 16
// and channels (l / 16) * S + s at step s, so each lane reads one contiguous
// run of S channels of its row (vector loads, issued before the chain); W is
// staged once per block in LDS (rows padded by 4 floats) and read in the same
// channel order.
__host__ __device__ inline int label_stride(int n_lab) { return n_lab + ((4 - n_lab % 16) + 16) % 16; }

template <int S, typename T>
__device__ inline void load_run(const T *p, float (&a)[S]) {
  if constexpr (sizeof(T) == 4 && S % 4 == 0) {
#pragma unroll
    for (int i = 0; i < S / 4; ++i) {
      const float4 v = reinterpret_cast<const float4 *>(p)[i];
      a[4 * i] = v.x;
      a[4 * i + 1] = v.y;
      a[4 * i + 2] = v.z;
      a[4 * i + 3] = v.w;
    }
  } else if constexpr (sizeof(T) == 2 && S % 8 == 0) {
    // bf16: eight channels per 16-byte load (a run starts at a multiple of S
    // channels of a row of K C, so it is 16-byte aligned)
#pragma unroll
    for (int i = 0; i < S / 8; ++i) {
      const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        a[8 * i + 2 * h] = __uint_as_float(w[h] << 16);
        a[8 * i + 2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < S; ++i) a[i] = Store<T>::ld(p + i);
  }
}

// NW waves per workgroup share the staged template and weights; each wave has
// its own label tile, so large shell lists (g shells: 625 labels per row) run
// with fewer waves per workgroup to fit in LDS.
template <int S, int NW, typename T>
__global__ void __launch_bounds__(kWave * NW) hblocks_kernel(int slot, int64_t rows, const T *__restrict__ irreps,
                                                              int K, const float *__restrict__ W, int n_w,
                                                              int n_lab, int n_ent, float *__restrict__ H) {
  constexpr int kWaves = NW;
  constexpr int C = 4 * S;
  constexpr int WLD = C + 4;  // padded LDS row of W
  extern __shared__ float smem[];
  const Table &tb = g_tables[slot];
  const int n_terms = tb.term_start[n_ent];
  // every piece is addressed from smem by an index: a round trip through an
  // integer address would lose the LDS address space and turn the reads into
  // flat loads, which wait on global memory traffic too
  int *t_start = reinterpret_cast<int *>(smem);                        // [n_ent + 1]
  float *t_coef = smem + (n_ent + 1);                                  // [n_terms]
  int *t_idx = reinterpret_cast<int *>(t_coef + n_terms);              // [n_terms]
  float *wl = smem + ((n_ent + 1 + 2 * n_terms + 3) & ~3);             // [n_w + 16][WLD], 16-byte aligned (zero rows after n_w)
  // label rows padded to lab_ld = 4 (mod 16) floats: the four 16-lane groups
  // of an MFMA result store then land on disjoint LDS bank ranges
  const int lab_ld = label_stride(n_lab);
  float *hs_all = wl + (n_w + 16) * WLD;                               // [kWaves][kTile][lab_ld]
  // per-degree entries of the table, read once per (tile, L) in the label loop
  __shared__ int l_n[kMaxLabL + 1], l_woff[kMaxLabL + 1], l_hoff[kMaxLabL + 1];
  if (threadIdx.x <= kMaxLabL) {
    l_n[threadIdx.x] = tb.nL[threadIdx.x];
    l_woff[threadIdx.x] = tb.woff[threadIdx.x];
    l_hoff[threadIdx.x] = tb.hoff[threadIdx.x];
  }
  for (int i = threadIdx.x; i <= n_ent; i += blockDim.x) t_start[i] = tb.term_start[i];
  for (int i = threadIdx.x; i < n_terms; i += blockDim.x) {
    t_coef[i] = tb.term_coef[i];
    t_idx[i] = tb.term_idx[i];
  }
  for (int i = threadIdx.x; i < (n_w + 16) * WLD; i += blockDim.x) {
    const int r = i / WLD, c = i - r * WLD;
    wl[i] = (r < n_w && c < C) ? W[static_cast<int64_t>(r) * C + c] : 0.0f;
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  float *hs = hs_all + wave * kTile * lab_ld;
  const int grp = lane / 16, i16 = lane % 16;
  const int lmax_lab = tb.lmax_lab;
  const int n_runs = (lmax_lab + 1) * (lmax_lab + 1);  // (L, M) runs of a row, in L^2 + L + M order
  const int64_t n_tiles = (rows + kTile - 1) / kTile;
  auto row_of = [&](int64_t tile) {
    const int64_t ea = min(tile * kTile + i16, rows - 1);  // clamped row for loads
    return irreps + ea * K * C + grp * S;
  };
  // The runs of this wave's tiles form one sequence (tile, run r of the tile,
  // its degree L and order M), stepped one run at a time without divisions.
  // Run k + 1 loads while run k multiplies, into the other of two named
  // buffers (the loop is unrolled by two, so no register copies), and a tile's
  // entries are formed after its last run, while the next tile's first run is
  // in flight.
  struct Pos {
    int64_t tile;
    int r, L, M;
  };
  auto next = [&](Pos p) {
    if (++p.r == n_runs) return Pos{p.tile + static_cast<int64_t>(gridDim.x) * kWaves, 0, 0, 0};
    if (++p.M > p.L) {
      ++p.L;
      p.M = -p.L;
    }
    return p;
  };
  // unconditional (past the last tile row_of clamps to the last row, and the
  // run is never used): a branch here would make the compiler wait for every
  // load in flight before each MFMA chain
  auto issue = [&](const Pos &p, float(&dst)[S]) { load_run<S>(row_of(p.tile) + p.r * C, dst); };
  auto run = [&](const Pos &p, const float(&a)[S]) {
    const int L = p.L, M = p.M;
    const int nL = l_n[L];
    const int ntile = (nL + 15) / 16;
    const int woff = l_woff[L], hoff = l_hoff[L];
    bool valu = false;
    if constexpr (S >= 32) valu = nL <= kValuLabels;
    if (valu) {
      // a few label channels of a wide row: dot products on the VALU (an MFMA
      // tile would compute 16 columns for them), each lane over its run of S
      // channels, then the four channel groups of a row summed across lanes.
      // (At S = 16 the 16-step MFMA chain was the faster of the two.)
      for (int k = 0; k < nL; ++k) {
        const float *wrow = wl + (woff + k) * WLD + grp * S;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < S; ++i) part += a[i] * wrow[i];
        part += __shfl_xor(part, 16, kWave);
        part += __shfl_xor(part, 32, kWave);
        if (grp == 0) hs[i16 * lab_ld + hoff + (M + L) * nL + k] = part;
      }
    } else {
      for (int t = 0; t < ntile; ++t) {
        // rows beyond n_L read the zero rows of the pad (or the next L's rows, discarded below)
        const float *brow = wl + (woff + 16 * t + i16) * WLD + grp * S;
        float b[S];
#pragma unroll
        for (int i = 0; i < S; ++i) b[i] = brow[i];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < S; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
        // D[i][j]: row i = 4 * (lane / 16) + rr, column j = lane % 16
        const int k = 16 * t + i16;
        if (k < nL) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) hs[(4 * grp + rr) * lab_ld + hoff + (M + L) * nL + k] = acc[rr];
        }
      }
    }
    if (p.r == n_runs - 1) {  // the tile's labels are complete: its entries
      // lane = entry, eight rows of the tile at a time, so each term's
      // coefficient and label index are read once per eight rows
      constexpr int R = 8;
      const int64_t e0 = p.tile * kTile;
      const int nrow = static_cast<int>(min(static_cast<int64_t>(kTile), rows - e0));
      wave_lds_order();
      for (int ent = lane; ent < n_ent; ent += kWave) {
        const int t0 = t_start[ent], t1 = t_start[ent + 1];
        for (int r0 = 0; r0 < nrow; r0 += R) {
          float acc[R];
#pragma unroll
          for (int el = 0; el < R; ++el) acc[el] = 0.0f;
#pragma unroll 1
          for (int t = t0; t < t1; ++t) {
            const float cf = t_coef[t];
            const int ix = t_idx[t];
#pragma unroll
            for (int el = 0; el < R; ++el) acc[el] += cf * hs[(r0 + el) * lab_ld + ix];
          }
#pragma unroll
          for (int el = 0; el < R; ++el)
            if (r0 + el < nrow) H[(e0 + r0 + el) * n_ent + ent] = acc[el];
        }
      }
      wave_lds_order();
    }
  };
  float a0[S], a1[S];
  Pos p0{static_cast<int64_t>(blockIdx.x) * kWaves + wave, 0, 0, 0};
  issue(p0, a0);
  while (p0.tile < n_tiles) {
    const Pos p1 = next(p0);
    issue(p1, a1);
    run(p0, a0);
    if (p1.tile >= n_tiles) break;
    p0 = next(p1);
    issue(p0, a0);
    run(p1, a1);
  }
}

template <int S, typename T>
void launch_hblocks_nw(int nw, unsigned g, size_t smem, hipStream_t stream, int slot, int64_t rows, const T *irr,
                       int K, const float *W, int n_w, int n_lab, int n_ent, float *H) {
  if (nw == 8)
    hblocks_kernel<S, 8, T><<<g, kWave * 8, smem, stream>>>(slot, rows, irr, K, W, n_w, n_lab, n_ent, H);
  else if (nw == 4)
    hblocks_kernel<S, 4, T><<<g, kWave * 4, smem, stream>>>(slot, rows, irr, K, W, n_w, n_lab, n_ent, H);
  else if (nw == 2)
    hblocks_kernel<S, 2, T><<<g, kWave * 2, smem, stream>>>(slot, rows, irr, K, W, n_w, n_lab, n_ent, H);
  else
    hblocks_kernel<S, 1, T><<<g, kWave * 1, smem, stream>>>(slot, rows, irr, K, W, n_w, n_lab, n_ent, H);
}

template <typename T>
egnn_status launch_hblocks(int slot, int64_t rows, const void *irreps, int K, int C, const float *W, int n_w,
                           int n_lab, int n_ent, int n_terms, float *H, hipStream_t stream) {
  if (rows <= 0) return EGNN_OK;
  auto smem_for = [&](int nw) {
    return sizeof(float) * (static_cast<size_t>(n_ent + 1) + 2 * n_terms + 4 + static_cast<size_t>(n_w + 16) * (C + 4) +
                            static_cast<size_t>(nw) * kTile * label_stride(n_lab));
  };
  // Waves per workgroup: the count that puts the most waves on a CU, where a
  // CU's 160 KB of LDS holds whole workgroups (the staged weights are shared
  // by a workgroup's waves, the label tiles are per wave).  Four waves win
  // ties.  At C 128 the weights take ~32 KB, so four waves (84 KB) leave room
  // for one workgroup and eight (130 KB) put twice the waves on the CU.
  constexpr size_t kCuLds = 160 * 1024, kMaxLds = 150 * 1024;
  int nw = 0;
  size_t best = 0;
  for (const int c : {4, 8, 2, 1}) {
    const size_t sm = smem_for(c);
    if (sm > kMaxLds) continue;
    const size_t waves = static_cast<size_t>(c) * (kCuLds / sm);
    if (waves > best) {
      best = waves;
      nw = c;
    }
  }
  if (nw == 0) {
    set_error("decode needs %zu bytes of LDS; reduce C or the shell list", smem_for(1));
    return EGNN_E_UNSUPPORTED;
  }
  const size_t smem = smem_for(nw);
  Timed t(stream, "hblocks", 0.0,
          double(rows) * (double(K) * C * sizeof(T) + double(n_ent) * 4.0) + double(C) * n_w * 4.0);
  int64_t blocks = ((rows + kTile - 1) / kTile + nw - 1) / nw;
  if (blocks > 2048 * 4 / nw) blocks = 2048 * 4 / nw;
  const unsigned g = static_cast<unsigned>(blocks);
  const T *irr = static_cast<const T *>(irreps);
  switch (C) {
    case 8: launch_hblocks_nw<2, T>(nw, g, smem, stream, slot, rows, irr, K, W, n_w, n_lab, n_ent, H); break;
    case 16: launch_hblocks_nw<4, T>(nw, g, smem, stream, slot, rows, irr, K, W, n_w, n_lab, n_ent, H); break;
    case 32: launch_hblocks_nw<8, T>(nw, g, smem, stream, slot, rows, irr, K, W, n_w, n_lab, n_ent, H); break;
    case 64: launch_hblocks_nw<16, T>(nw, g, smem, stream, slot, rows, irr, K, W, n_w, n_lab, n_ent, H); break;
    case 128: launch_hblocks_nw<32, T>(nw, g, smem, stream, slot, rows, irr, K, W, n_w, n_lab, n_ent, H); break;
    case 256: launch_hblocks_nw<64, T>(nw, g, smem, stream, slot, rows, irr, K, W, n_w, n_lab, n_ent, H); break;
    default:
      set_error("decode supports C in {8, 16, 32, 64, 128, 256}");
      return EGNN_E_UNSUPPORTED;
  }
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}

// Periodic assembly, in two passes.  Pass 1 (one wave per block row = source
// atom) writes the row pointers, columns and shifts.  The row's blocks are
// its source group's edges, already in ascending (destination, shift) order
// because edge ids run destination-major and each destination row is sorted
// by (source, shift), plus the on-site block of an owned atom, placed where
// (i, 0, 0, 0) falls in that order: an edge lands one slot later when it
// sorts after the on-site block, and the on-site block's slot is the count of
// edges that sort before it.  Pass 2 copies the values: each wave takes
// kBsrChunk consecutive output blocks (one contiguous output range), finds
// each block's input from the columns and shifts of pass 1, and streams the
// range with several independent loads per lane in flight.
__device__ inline int dst_of_edge(const int *row_ptr, int n_dst, int e) {
  int lo = 0, hi = n_dst;  // largest d with row_ptr[d] <= e
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row_ptr[mid] <= e) lo = mid; else hi = mid;
  }
  return lo;
}

// (col, s) after (i, 0, 0, 0) in (destination, S_x, S_y, S_z) order
__device__ inline bool after_onsite(int col, int s0, int s1, int s2, int i) {
  return col > i || (col == i && (s0 > 0 || (s0 == 0 && (s1 > 0 || (s1 == 0 && s2 > 0)))));
}

__global__ void __launch_bounds__(256) bsr_index_kernel(const int *__restrict__ row_ptr, int n_dst,
                                                        const int *__restrict__ src_ptr,
                                                        const int *__restrict__ src_perm,
                                                        const int8_t *__restrict__ shift, int n_src, int64_t E,
                                                        bool onsite, int *__restrict__ brp, int *__restrict__ bcol,
                                                        int8_t *__restrict__ bsh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  if (i >= n_src) return;
  const int g0 = src_ptr[i], cnt = src_ptr[i + 1] - g0;
  const bool on = onsite && i < n_dst;
  const int64_t base = g0 + (onsite ? min(i, n_dst) : 0);
  if (lane == 0) {
    brp[i] = static_cast<int>(base);
    if (i == n_src - 1) brp[n_src] = static_cast<int>(E + (onsite ? n_dst : 0));
  }
  int before = 0;  // edges of the group ordered before (i, 0, 0, 0)
  for (int t0 = 0; t0 < cnt; t0 += kWave) {
    const int t = t0 + lane;
    bool lt = false;
    if (t < cnt) {
      const int e = src_perm[g0 + t];
      const int d = dst_of_edge(row_ptr, n_dst, e);
      const int8_t *sv = shift + 3 * static_cast<int64_t>(e);
      const int s0 = sv[0], s1 = sv[1], s2 = sv[2];
      const bool late = on && after_onsite(d, s0, s1, s2, i);
      lt = on && !late;
      const int64_t u = base + t + (late ? 1 : 0);
      bcol[u] = d;
      int8_t *o = bsh + 3 * u;
      o[0] = static_cast<int8_t>(s0);
      o[1] = static_cast<int8_t>(s1);
      o[2] = static_cast<int8_t>(s2);
    }
    before += __popcll(__ballot(lt));
  }
  if (on && lane == 0) {
    const int64_t u = base + before;
    bcol[u] = i;
    bsh[3 * u] = 0;
    bsh[3 * u + 1] = 0;
    bsh[3 * u + 2] = 0;
  }
}

constexpr int kBsrChunk = 16;  // output blocks per wave in the value pass
constexpr int kBsrLoads = 8;   // loads in flight per lane

__global__ void __launch_bounds__(256) bsr_values_kernel(const int *__restrict__ brp, int n_src, int n_dst,
                                                         const int *__restrict__ src_ptr,
                                                         const int *__restrict__ src_perm,
                                                         const int *__restrict__ bcol,
                                                         const int8_t *__restrict__ bsh, int64_t nnzb, int nb2,
                                                         const float *__restrict__ h_edge,
                                                         const float *__restrict__ h_onsite,
                                                         float *__restrict__ bval) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave * kBsrChunk;
  if (b0 >= nnzb) return;
  const int nb = static_cast<int>(min(static_cast<int64_t>(kBsrChunk), nnzb - b0));
  // lanes 0..nb-1: the input block of output block b0 + lane
  int64_t src_blk = 0;  // element offset of the input block; on-site blocks are tagged by the sign
  if (lane < nb) {
    const int b = static_cast<int>(b0 + lane);
    int lo = 0, hi = n_src;  // row: largest i with brp[i] <= b
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (brp[mid] <= b) lo = mid; else hi = mid;
    }
    const int i = lo, u = b - brp[i];
    const int col = bcol[b];
    const int s0 = bsh[3 * static_cast<int64_t>(b)], s1 = bsh[3 * static_cast<int64_t>(b) + 1],
              s2 = bsh[3 * static_cast<int64_t>(b) + 2];
    const bool on = h_onsite != nullptr && i < n_dst;
    if (on && col == i && s0 == 0 && s1 == 0 && s2 == 0) {
      src_blk = -1 - static_cast<int64_t>(i) * nb2;
    } else {
      const int t = u - ((on && after_onsite(col, s0, s1, s2, i)) ? 1 : 0);
      src_blk = static_cast<int64_t>(src_perm[src_ptr[i] + t]) * nb2;
    }
  }
  const int total = nb * nb2;
  float *out = bval + b0 * nb2;
  for (int o0 = 0; o0 < total; o0 += kWave * kBsrLoads) {
    float v[kBsrLoads];
#pragma unroll
    for (int k = 0; k < kBsrLoads; ++k) {
      const int o = o0 + k * kWave + lane;
      const int blk = o / nb2, r = o - blk * nb2;
      const int64_t sb = __shfl(src_blk, min(blk, kBsrChunk - 1));
      v[k] = 0.0f;
      if (o < total) v[k] = sb >= 0 ? h_edge[sb + r] : h_onsite[-1 - sb + r];
    }
#pragma unroll
    for (int k = 0; k < kBsrLoads; ++k) {
      const int o = o0 + k * kWave + lane;
      if (o < total) out[o] = v[k];
    }
  }
}

}  // namespace
}  // namespace egnn

using namespace egnn;

extern "C" egnn_status egnn_assemble_bsr(const egnn_graph *g, int32_t n_orb, const float *h_edge,
                                         const float *h_onsite, int32_t *bsr_row_ptr, int32_t *bsr_col,
                                         int8_t *bsr_shift, float *bsr_val, hipStream_t stream) {
  clear_error();
  EGNN_REQUIRE(g, "graph is null");
  EGNN_REQUIRE(g->n_dst >= 0 && g->n_src >= g->n_dst, "need 0 <= n_dst <= n_src");
  EGNN_REQUIRE(g->n_edges >= 0 && g->n_edges <= g->capacity, "graph n_edges out of range");
  EGNN_REQUIRE(n_orb >= 1 && n_orb <= kMaxOrb, "n_orb must be 1..%d", kMaxOrb);
  const int64_t nnzb = g->n_edges + (h_onsite ? g->n_dst : 0);
  EGNN_REQUIRE(nnzb <= INT32_MAX, "more than 2^31 - 1 blocks");
  EGNN_REQUIRE(bsr_row_ptr && g->src_ptr, "row pointers are null");
  if (g->n_src == 0) return EGNN_OK;
  if (g->n_edges > 0)
    EGNN_REQUIRE(h_edge && g->row_ptr && g->src_perm && g->shift, "edge pointers are null");
  if (nnzb > 0) EGNN_REQUIRE(bsr_col && bsr_shift && bsr_val, "block arrays are null");
  const int nb2 = n_orb * n_orb;
  Timed t(stream, "assemble_bsr", 0.0, double(nnzb) * (2.0 * 4.0 * nb2 + 4.0 + 3.0 + 8.0) + 4.0 * g->n_src);
  const int T = 256;
  bsr_index_kernel<<<ceil_div(static_cast<int64_t>(g->n_src) * kWave, T), T, 0, stream>>>(
      g->row_ptr, g->n_dst, g->src_ptr, g->src_perm, g->shift, g->n_src, g->n_edges, h_onsite != nullptr,
      bsr_row_ptr, bsr_col, bsr_shift);
  EGNN_CHECK_LAUNCH();
  if (nnzb > 0) {
    bsr_values_kernel<<<ceil_div(ceil_div(nnzb, kBsrChunk) * kWave, T), T, 0, stream>>>(
        bsr_row_ptr, g->n_src, g->n_dst, g->src_ptr, g->src_perm, bsr_col, bsr_shift, nnzb, nb2, h_edge, h_onsite,
        bsr_val);
    EGNN_CHECK_LAUNCH();
  }
  return EGNN_OK;
}

static bool valid_hdesc(const egnn_hdesc *h) {
  if (!h || !h->shell_l) return false;
  if (h->n_shells < 1 || h->n_shells > 16) return false;
  if (h->lmax < 0 || h->lmax > 8) return false;
  if (h->C < 8 || h->C > 256 || (h->C & (h->C - 1)) != 0) return false;  // C/4 channel steps per lane group
  if (h->storage != EGNN_F32 && h->storage != EGNN_BF16) return false;
  int lmx = 0;
  for (int i = 0; i < h->n_shells; ++i) {
    if (h->shell_l[i] < 0 || h->shell_l[i] > kMaxShellL) return false;
    lmx = std::max(lmx, h->shell_l[i]);
  }
  return h->lmax >= 2 * lmx;
}

extern "C" int32_t egnn_hblocks_label_rows(const egnn_hdesc *h) {
  if (!valid_hdesc(h)) return 0;
  Layout lay;
  if (!build_layout(h->shell_l, h->n_shells, &lay)) return 0;
  return lay.n_w;
}

extern "C" egnn_status egnn_hblocks(const egnn_hdesc *h, int64_t n_edges, int32_t n_nodes, const float *w_edge,
                                    const float *w_node, const void *edge_irreps, const void *node_irreps,
                                    float *h_edge, float *h_onsite, hipStream_t stream) {
  clear_error();
  EGNN_REQUIRE(valid_hdesc(h), "invalid decode description");
  EGNN_REQUIRE(n_edges >= 0 && n_nodes >= 0, "negative row count");
  if (n_edges > 0) EGNN_REQUIRE(w_edge && edge_irreps && h_edge, "edge pointers are null");
  if (n_nodes > 0) EGNN_REQUIRE(w_node && node_irreps && h_onsite, "node pointers are null");
  // each lane reads its channel run with 16-byte loads
  auto aligned16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (n_edges > 0) EGNN_REQUIRE(aligned16(edge_irreps), "edge irreps must be 16-byte aligned");
  if (n_nodes > 0) EGNN_REQUIRE(aligned16(node_irreps), "node irreps must be 16-byte aligned");
  if (n_edges == 0 && n_nodes == 0) return EGNN_OK;
  int slot = 0;
  Layout lay;
  egnn_status st = table_slot(h->shell_l, h->n_shells, &slot, &lay);
  if (st != EGNN_OK) return st;
  const int K = (h->lmax + 1) * (h->lmax + 1);
  const int n_ent = lay.n_orb * lay.n_orb;
  auto run = [&](int64_t rows, const void *irr, const float *W, float *H) -> egnn_status {
    if (h->storage == EGNN_BF16)
      return launch_hblocks<uint16_t>(slot, rows, irr, K, h->C, W, lay.n_w, lay.n_lab, n_ent, lay.t.term_start[n_ent], H,
                                      stream);
    return launch_hblocks<float>(slot, rows, irr, K, h->C, W, lay.n_w, lay.n_lab, n_ent, lay.t.term_start[n_ent], H,
                                 stream);
  };
  st = run(n_edges, edge_irreps, w_edge, h_edge);
  if (st != EGNN_OK) return st;
  return run(n_nodes, node_irreps, w_node, h_onsite);
}
