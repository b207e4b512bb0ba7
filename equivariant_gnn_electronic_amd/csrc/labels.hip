// Matrix <-> Label over whole Hamiltonian matrices (MALOQ Sec. III-B2).
//
// A batch holds one dense row-major matrix per structure, back to back.  Each
// element carries a subset of one full shell list (its orbital template); an
// atom's orbitals are its shells in full-list order, m = -l..l each, and its
// first orbital is the sum of the orbital counts of the atoms before it in
// its structure.  Matrix -> Label cuts the block of every node (on-site) and
// edge (rows = source orbitals, columns = destination orbitals) into a buffer
// of the full list's shape, zero where the template has no orbital, and
// applies Eq. (1) of Sec. III-B1 to every shell pair.  Label q = (L, M,
// k(a, b, L)) follows the full list's layout, so the labels of shell pairs an
// element lacks are zero: they are the padding to the largest element.  Label
// -> Matrix applies the transpose and writes the template's entries back.
//
// The pages' CUDA kernel gives one thread per matrix element and one thread
// block per node or edge, driven by an orbital template per element pair.
// Here the templates are the distinct shell masks of the elements, and the
// host builds, for every ordered template pair, the CG terms of exactly the
// labels and entries that pair carries.  One 64-lane wave owns a destination
// row.  It describes the row's blocks (its on-site block, then its edges) 64
// at a time, one per lane, groups them by template pair, and takes each
// group CB blocks at a time: their present entries (or labels) are loaded
// with CB independent loads per lane in flight and staged in LDS, then lanes
// run over the pair's outputs, dealt to them by term count so that every
// lane of a pass runs the same number of terms, and each term is read once
// for all CB blocks.  Labels a pair lacks are written as zeros.  The next
// chunk's loads are issued before the current chunk's outputs are formed.
#include <algorithm>
#include <climits>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "cg_real.h"
#include "common.h"
#include "timing.h"

namespace egnn {
namespace {

constexpr int kLSlots = 4;
constexpr int kFullMax = 32;                 // orbitals of the full shell list
constexpr int kSpeciesMax = 64;
constexpr int kShellLMax = 4;                // s, p, d, f, g shells: labels up to L = 8
constexpr int kTmplMax = 8;                  // distinct element bases (shell masks)
constexpr int kPairN = (kTmplMax + 1) * (kTmplMax + 1);  // ordered template pairs, the empty template included
constexpr int kRowMax = 2048;                // padded term rows per direction
constexpr int kPosMax = 1 << 15;             // lane outputs over all passes
constexpr int kPassTot = 4096;               // passes over all pairs and both directions

// Per ordered template pair (u: source / row side, w: destination / column
// side).  The pair's own block is n_u x n_w, its entries p = lr * n_w + lc;
// it carries P = n_u * n_w of the labels (one per own entry).
struct PairInfo {
  int P, n_w, magic;        // present entries; columns; ceil(2^16 / n_w) (p / n_w = p * magic >> 16, p < 2048)
  int lpass, lprow, lpos;   // Matrix -> Label: passes over the present labels (pos: label q)
  int zpass, zpos;          //   passes over the absent labels (pos: label q, written as zero)
  int spass, spos;          // Label -> Matrix: staging passes (pos: label q of compact input i)
  int epass, eprow, epos;   //   passes over the own entries (pos: entry p)
};
constexpr int kPairInts = sizeof(PairInfo) / sizeof(int);

// Padded lane-major passes: pass ps of a pair reads term rows
// prow[xprow + ps] .. prow[xprow + ps + 1] - 1, lane l taking coef / idx
// [row][l] (zero coefficients pad the shorter term lists), and writes output
// pos[xpos + ps * 64 + l] (-1: none).
struct LabelTable {
  int n_full, n_lab, n_species, n_tmpl;
  int n_orb[kSpeciesMax];                    // orbitals of each element
  int tmpl[kSpeciesMax];                     // template of each element
  PairInfo pair[kPairN];                     // [u * (n_tmpl + 1) + w], template n_tmpl = empty
  int n_prow, n_pos, rows[2];                // used sizes; rows per direction (0: to labels, 1: to entries)
  int prow[kPassTot];
  int16_t pos[kPosMax];
  float coef[2][kRowMax * 64];
  uint16_t idx[2][kRowMax * 64];
};

__device__ LabelTable g_ltables[kLSlots];

// Builds the table; returns nullptr, or why the basis is not accepted.
const char *build_label_table(const egnn_basis *b, LabelTable *t) {
  if (!b || !b->shell_l || !b->species_shells) return "basis pointers are null";
  if (b->n_shells < 1 || b->n_shells > 16) return "n_shells must be 1..16";
  if (b->n_species < 1 || b->n_species > kSpeciesMax) return "n_species must be 1..64";
  const int ns = b->n_shells;
  std::vector<int> off(ns);
  int o = 0, lmx = 0;
  for (int a = 0; a < ns; ++a) {
    const int l = b->shell_l[a];
    if (l < 0 || l > kShellLMax) return "shell degrees must be 0..4";
    off[a] = o;
    o += 2 * l + 1;
    lmx = std::max(lmx, l);
  }
  if (o > kFullMax) return "the full shell list has more than 32 orbitals";
  for (int z = 0; z < b->n_species; ++z)
    if (b->species_shells[z] >> ns) return "a species mask names a shell beyond n_shells";
  std::memset(t, 0, sizeof(*t));
  t->n_full = o;
  t->n_lab = o * o;
  t->n_species = b->n_species;
  // templates: the distinct masks, in order of first appearance
  std::vector<uint32_t> masks;
  for (int z = 0; z < b->n_species; ++z) {
    const uint32_t m = b->species_shells[z];
    int u = static_cast<int>(std::find(masks.begin(), masks.end(), m) - masks.begin());
    if (u == static_cast<int>(masks.size())) {
      if (u >= kTmplMax) return "more than 8 distinct element bases";
      masks.push_back(m);
    }
    t->tmpl[z] = u;
  }
  const int T = static_cast<int>(masks.size());
  t->n_tmpl = T;
  masks.push_back(0u);  // the empty template
  // own orbital of each full orbital, per template (-1 if absent)
  std::vector<std::vector<int>> omap(T + 1, std::vector<int>(o, -1));
  std::vector<int> norb(T + 1, 0);
  for (int u = 0; u <= T; ++u)
    for (int a = 0; a < ns; ++a)
      if ((masks[u] >> a) & 1u)
        for (int m = 0; m < 2 * b->shell_l[a] + 1; ++m) omap[u][off[a] + m] = norb[u]++;
  for (int z = 0; z < b->n_species; ++z) t->n_orb[z] = norb[t->tmpl[z]];
  // label channels of the full list: ordered shell pairs, L ascending
  const int Lmax = 2 * lmx;
  std::vector<int> nL(Lmax + 1, 0), hoff(Lmax + 2, 0);
  struct Item { int a, b, L, k; };
  std::vector<Item> items;
  for (int a = 0; a < ns; ++a)
    for (int c = 0; c < ns; ++c)
      for (int L = std::abs(b->shell_l[a] - b->shell_l[c]); L <= b->shell_l[a] + b->shell_l[c]; ++L)
        items.push_back({a, c, L, nL[L]++});
  for (int L = 0; L <= Lmax; ++L) hoff[L + 1] = hoff[L] + (2 * L + 1) * nL[L];
  if (hoff[Lmax + 1] != o * o) return "internal: label count differs from the block size";
  std::vector<std::vector<double>> Q(items.size());
  for (size_t it = 0; it < items.size(); ++it)
    Q[it] = cg::real_coupling(b->shell_l[items[it].a], b->shell_l[items[it].b], items[it].L);
  typedef std::vector<std::pair<float, int>> Terms;
  // deal outputs (id, terms) to padded lane-major passes of direction d
  auto deal = [&](const std::vector<std::pair<int, Terms>> &outs, int d, int *npass, int *prow0, int *pos0) {
    const int n = static_cast<int>(outs.size());
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return outs[x].second.size() > outs[y].second.size(); });
    *npass = (n + 63) / 64;
    *prow0 = t->n_prow;
    *pos0 = t->n_pos;
    if (t->n_prow + *npass + 1 > kPassTot || t->n_pos + 64 * *npass > kPosMax) return false;
    for (int ps = 0; ps < *npass; ++ps) {
      size_t iters = 0;
      for (int l = 0; l < 64; ++l) {
        const int k = ps * 64 + l;
        t->pos[t->n_pos + k] = static_cast<int16_t>(k < n ? outs[order[k]].first : -1);
        if (k < n) iters = std::max(iters, outs[order[k]].second.size());
      }
      t->prow[t->n_prow + ps] = t->rows[d];
      if (t->rows[d] + static_cast<int>(iters) > kRowMax) return false;
      for (size_t it = 0; it < iters; ++it, ++t->rows[d])
        for (int l = 0; l < 64; ++l) {
          const int k = ps * 64 + l;
          const bool has = k < n && it < outs[order[k]].second.size();
          t->coef[d][t->rows[d] * 64 + l] = has ? outs[order[k]].second[it].first : 0.0f;
          t->idx[d][t->rows[d] * 64 + l] = static_cast<uint16_t>(has ? outs[order[k]].second[it].second : 0);
        }
    }
    t->prow[t->n_prow + *npass] = t->rows[d];
    t->n_prow += *npass + 1;
    t->n_pos += 64 * *npass;
    return true;
  };
  auto plain = [&](const std::vector<int> &ids, int *npass, int *pos0) {
    *npass = (static_cast<int>(ids.size()) + 63) / 64;
    *pos0 = t->n_pos;
    if (t->n_pos + 64 * *npass > kPosMax) return false;
    for (int k = 0; k < 64 * *npass; ++k)
      t->pos[t->n_pos + k] = static_cast<int16_t>(k < static_cast<int>(ids.size()) ? ids[k] : -1);
    t->n_pos += 64 * *npass;
    return true;
  };
  for (int u = 0; u <= T; ++u)
    for (int w = 0; w <= T; ++w) {
      PairInfo &pi = t->pair[u * (T + 1) + w];
      pi.P = norb[u] * norb[w];
      pi.n_w = std::max(norb[w], 1);
      pi.magic = (65536 + pi.n_w - 1) / pi.n_w;
      // labels the pair carries, with their terms over own entries p
      std::vector<std::pair<int, Terms>> labs;
      std::vector<int> absent;
      std::vector<std::vector<std::pair<float, int>>> by_ent(pi.P);
      std::vector<int> present_q;
      for (size_t it = 0; it < items.size(); ++it) {
        const Item &im = items[it];
        const int la = b->shell_l[im.a], lb = b->shell_l[im.b], nb = 2 * lb + 1, nm = 2 * im.L + 1;
        const bool has = ((masks[u] >> im.a) & 1u) && ((masks[w] >> im.b) & 1u);
        for (int M = 0; M < nm; ++M) {
          const int q = hoff[im.L] + M * nL[im.L] + im.k;
          if (!has) {
            absent.push_back(q);
            continue;
          }
          Terms tr;
          for (int i = 0; i < 2 * la + 1; ++i)
            for (int j = 0; j < nb; ++j) {
              const double c = Q[it][(i * nb + j) * nm + M];
              if (std::fabs(c) < 1e-12) continue;
              const int pe = omap[u][off[im.a] + i] * norb[w] + omap[w][off[im.b] + j];
              tr.push_back({static_cast<float>(c), pe});
            }
          labs.push_back({q, tr});
          present_q.push_back(q);
        }
      }
      std::sort(present_q.begin(), present_q.end());
      // Label -> Matrix: entries from the compact inputs i (labels in ascending q)
      for (size_t i = 0; i < present_q.size(); ++i)
        for (const auto &lq : labs)
          if (lq.first == present_q[i])
            for (const auto &tm : lq.second) by_ent[tm.second].push_back({tm.first, static_cast<int>(i)});
      std::vector<std::pair<int, Terms>> ents;
      for (int pe = 0; pe < pi.P; ++pe) ents.push_back({pe, by_ent[pe]});
      if (!deal(labs, 0, &pi.lpass, &pi.lprow, &pi.lpos) || !plain(absent, &pi.zpass, &pi.zpos) ||
          !plain(present_q, &pi.spass, &pi.spos) || !deal(ents, 1, &pi.epass, &pi.eprow, &pi.epos))
        return "the basis needs more coupling terms than the table holds";
    }
  return nullptr;
}

struct LKey {
  int n_shells, n_species;
  int l[16];
  uint32_t mask[kSpeciesMax];
};
struct LInfo {
  int n_full, n_lab, n_species, n_tmpl, n_prow, n_pos, rows[2];
};
struct LCache {
  std::mutex mu;
  LKey keys[64][kLSlots];
  LInfo info[64][kLSlots];
  int used[64] = {0};
};
LCache g_lcache;

egnn_status label_slot(const egnn_basis *b, int *slot, LInfo *info) {
  int dev = 0;
  EGNN_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) {
    set_error("device index %d out of range", dev);
    return EGNN_E_UNSUPPORTED;
  }
  if (!b || !b->shell_l || !b->species_shells || b->n_shells < 1 || b->n_shells > 16 || b->n_species < 1 ||
      b->n_species > kSpeciesMax) {
    set_error("invalid basis description");
    return EGNN_E_ARG;
  }
  LKey key;
  std::memset(&key, 0, sizeof(key));
  key.n_shells = b->n_shells;
  key.n_species = b->n_species;
  std::memcpy(key.l, b->shell_l, sizeof(int) * b->n_shells);
  std::memcpy(key.mask, b->species_shells, sizeof(uint32_t) * b->n_species);
  std::lock_guard<std::mutex> lock(g_lcache.mu);
  for (int s = 0; s < g_lcache.used[dev]; ++s)
    if (std::memcmp(&g_lcache.keys[dev][s], &key, sizeof(key)) == 0) {
      *slot = s;
      *info = g_lcache.info[dev][s];
      return EGNN_OK;
    }
  std::vector<LabelTable> t(1);
  if (const char *why = build_label_table(b, t.data())) {
    set_error("basis not supported: %s", why);
    return EGNN_E_UNSUPPORTED;
  }
  if (g_lcache.used[dev] >= kLSlots) {
    set_error("more than %d distinct bases on one device", kLSlots);
    return EGNN_E_UNSUPPORTED;
  }
  const int s = g_lcache.used[dev];
  EGNN_TRY_HIP(hipMemcpyToSymbol(HIP_SYMBOL(g_ltables), t.data(), sizeof(LabelTable), sizeof(LabelTable) * s,
                                 hipMemcpyHostToDevice));
  g_lcache.keys[dev][s] = key;
  LInfo &in = g_lcache.info[dev][s];
  in.n_full = t[0].n_full;
  in.n_lab = t[0].n_lab;
  in.n_species = t[0].n_species;
  in.n_tmpl = t[0].n_tmpl;
  in.n_prow = t[0].n_prow;
  in.n_pos = t[0].n_pos;
  in.rows[0] = t[0].rows[0];
  in.rows[1] = t[0].rows[1];
  g_lcache.used[dev] = s + 1;
  *slot = s;
  *info = in;
  return EGNN_OK;
}

constexpr int kLW = 64;
constexpr int kLWaves = 16;

__global__ void fill_i32(int *p, int64_t n, int v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void zero_u64(unsigned long long *p) { *p = 0ull; }

// Source-grouped order: an edge whose source is no atom is in no group, so the
// main kernel never meets it.  It is a skipped block: counted here, and in
// Matrix -> Label its label row is zeroed here.
__global__ void __launch_bounds__(256) ungrouped_kernel(const int *__restrict__ src, int n_edges, int n_atoms,
                                                        int n_lab, float *__restrict__ lab_e_out,
                                                        unsigned long long *skipped) {
  const int lane = threadIdx.x & (kLW - 1);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  bool bad = false;
  if (e < n_edges) {
    const int s = src[e];
    bad = s < 0 || s >= n_atoms;
  }
  const unsigned long long m = __ballot(bad);
  if (lane == 0 && m && skipped) atomicAdd(skipped, static_cast<unsigned long long>(__popcll(m)));
  if (lab_e_out) {
    unsigned long long rem = m;
    while (rem) {  // the wave zeroes each such row together
      const int l = __ffsll(rem) - 1;
      rem &= rem - 1;
      const int64_t eb = static_cast<int64_t>(blockIdx.x) * blockDim.x + (threadIdx.x - lane) + l;
      for (int q = lane; q < n_lab; q += kLW) lab_e_out[eb * n_lab + q] = 0.0f;
    }
  }
}

// One wave per structure: each atom's first orbital is an exclusive scan of
// the orbital counts over the structure's atoms, 64 at a time.
__global__ void __launch_bounds__(256) layout_kernel(int slot, int n_mols, int n_atoms, const int *__restrict__ mol_ptr,
                                                     const int *__restrict__ species, int *__restrict__ atom_orb,
                                                     int *__restrict__ atom_mol, int *__restrict__ mol_norb,
                                                     unsigned long long *invalid) {
  const LabelTable &tb = g_ltables[slot];
  const int lane = threadIdx.x % kLW;
  const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kLW;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * blockDim.x / kLW;
  for (int64_t b = w0; b < n_mols; b += nw) {
    const int p0 = mol_ptr[b], p1 = mol_ptr[b + 1];
    if (!(p0 >= 0 && p0 <= p1 && p1 <= n_atoms)) {
      if (lane == 0) {
        mol_norb[b] = 0;
        if (invalid) atomicAdd(invalid, 1ull);
      }
      continue;
    }
    int run = 0;
    for (int a0 = p0; a0 < p1; a0 += kLW) {
      const int a = a0 + lane;
      int n = 0;
      bool bad = false;
      if (a < p1) {
        const int z = species[a];
        bad = !(z >= 0 && z < tb.n_species);
        n = bad ? 0 : tb.n_orb[z];
      }
      int incl = n;
#pragma unroll
      for (int d = 1; d < kLW; d <<= 1) {
        const int y = __shfl_up(incl, d, kLW);
        if (lane >= d) incl += y;
      }
      if (a < p1) {
        atom_orb[a] = run + incl - n;
        atom_mol[a] = static_cast<int>(b);
      }
      run += __shfl(incl, kLW - 1, kLW);
      const unsigned long long nbad = __popcll(__ballot(bad));
      if (lane == 0 && nbad && invalid) atomicAdd(invalid, nbad);
    }
    if (lane == 0) mol_norb[b] = run;
  }
}

// Exclusive scan of the matrix sizes n_b^2 over structures, one workgroup:
// each thread sums a contiguous run, the runs' sums are scanned in LDS.
__global__ void __launch_bounds__(1024) mat_off_kernel(int n_mols, const int *__restrict__ mol_norb,
                                                       int64_t *__restrict__ mat_off) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n_mols + 1023) / 1024;
  const int lo = min(tid * per, n_mols), hi = min(lo + per, n_mols);
  int64_t s = 0;
  for (int b = lo; b < hi; ++b) s += static_cast<int64_t>(mol_norb[b]) * mol_norb[b];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int64_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = part[tid] - s;
  for (int b = lo; b < hi; ++b) {
    mat_off[b] = run;
    run += static_cast<int64_t>(mol_norb[b]) * mol_norb[b];
  }
  if (tid == 1023) mat_off[n_mols] = part[1023];
}

struct Rows {
  int n_atoms, n_mols;
  const int *row_ptr, *src;
  const int8_t *shift;
  const int *src_ptr, *src_perm;  // grouped: the rows are source atoms, their blocks in src_perm order
  const int *mol_ptr;
  const int *species, *atom_orb, *atom_mol, *mol_norb;
  const int64_t *mat_off;
  int64_t h_elems;
  int n_edges;
  int nodes, edges;  // 1 = on-site blocks / edge blocks requested
  int grouped;
  int vec4;          // label rows are whole 16-byte units at 16-byte aligned addresses
};

// Block bi of row r: the on-site block first (when requested), then the
// row's edges.  By destination rows (r = j): edge row_ptr[j] + t, source
// src[e].  By source rows (r = i): edge src_perm[src_ptr[i] + t], whose
// destination is the row of the CSR that holds it, searched among the atoms
// of i's structure (an edge outside them has no block anyway).  A block with
// no place in a matrix gets the empty template pair (all labels zero,
// nothing written).
struct Blk {
  int64_t base, out;
  int ld, pair, node;
};

__device__ inline Blk block_of(const Rows &R, const LabelTable &tb, int64_t r, int bi, int e0, bool *ok_out) {
  const int T = tb.n_tmpl;
  Blk k;
  int i, j;
  bool ok = true;
  if (R.nodes && bi == 0) {
    i = j = static_cast<int>(r);
    k.node = 1;
    k.out = r;
  } else if (!R.grouped) {
    const int64_t e = static_cast<int64_t>(e0) + bi - R.nodes;
    j = static_cast<int>(r);
    i = R.src[e];
    k.node = 0;
    k.out = e;
  } else {
    const int e = R.src_perm[static_cast<int64_t>(e0) + bi - R.nodes];
    i = static_cast<int>(r);
    j = -1;
    ok = e >= 0 && e < R.n_edges;
    k.node = 0;
    k.out = ok ? e : 0;
    const int mi = R.atom_mol[i];
    if (ok && mi >= 0 && mi < R.n_mols) {
      const int a0 = min(max(R.mol_ptr[mi], 0), R.n_atoms);
      const int a1 = min(max(R.mol_ptr[mi + 1], a0), R.n_atoms);
      if (e >= R.row_ptr[a0] && e < R.row_ptr[a1]) {
        int lo = a0, hi = a1;  // the largest j < a1 with row_ptr[j] <= e
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (R.row_ptr[mid] <= e) lo = mid; else hi = mid;
        }
        j = lo;
      }
    }
  }
  ok = ok && i >= 0 && i < R.n_atoms && j >= 0 && j < R.n_atoms;
  if (!k.node && R.shift) {
    const int8_t *s = R.shift + 3 * k.out;
    ok = ok && s[0] == 0 && s[1] == 0 && s[2] == 0;
  }
  const int ic = ok ? i : 0;
  j = ok ? j : 0;
  const int mj = R.atom_mol[j], mi = R.atom_mol[ic];
  ok = ok && mj >= 0 && mj < R.n_mols && mi == mj;
  const int si = R.species[ic], sj = R.species[j];
  const int ui = (si >= 0 && si < tb.n_species) ? tb.tmpl[si] : T;
  const int uj = (sj >= 0 && sj < tb.n_species) ? tb.tmpl[sj] : T;
  const int ni = (si >= 0 && si < tb.n_species) ? tb.n_orb[si] : 0;
  const int nj = (sj >= 0 && sj < tb.n_species) ? tb.n_orb[sj] : 0;
  int ld = 0;
  int64_t mo = 0;
  if (ok) {  // only then is mj a structure (there may be none)
    ld = R.mol_norb[mj];
    mo = R.mat_off[mj];
  }
  const int oi = R.atom_orb[ic], oj = R.atom_orb[j];
  // (ld < 2^26 keeps the 32-bit entry offsets r * ld + c of the kernels exact)
  ok = ok && ld >= 0 && ld < (1 << 26) && oi >= 0 && oj >= 0 && oi + ni <= ld && oj + nj <= ld && mo >= 0 &&
       mo + static_cast<int64_t>(ld) * ld <= R.h_elems;
  *ok_out = ok;
  k.ld = ok ? ld : 0;
  k.base = ok ? mo + static_cast<int64_t>(oi) * ld + oj : 0;
  k.pair = ok ? ui * (T + 1) + uj : T * (T + 1) + T;
  return k;
}

// LDS words: pair table, pass rows, lane outputs (int16, two per word), one
// direction's term rows (coef, then idx as int16 pairs), then per wave CB
// staged blocks.
__host__ __device__ inline size_t lds_words(int n_pairs, int n_prow, int n_pos, int rows) {
  return (static_cast<size_t>(n_pairs) * kPairInts + n_prow + (n_pos + 1) / 2 + 64 * static_cast<size_t>(rows) +
          32 * static_cast<size_t>(rows) + 3) & ~static_cast<size_t>(3);
}

template <int CB, int NT, bool TO_LABEL>
__global__ void __launch_bounds__(kLW * kLWaves) labels_kernel(int slot, Rows R, const float *__restrict__ Hin,
                                                                float *__restrict__ Hout,
                                                                const float *__restrict__ lab_e_in,
                                                                const float *__restrict__ lab_n_in,
                                                                float *__restrict__ lab_e_out,
                                                                float *__restrict__ lab_n_out,
                                                                unsigned long long *skipped) {
  extern __shared__ float lsm[];
  const LabelTable &tb = g_ltables[slot];
  const int n_lab = tb.n_lab, T = tb.n_tmpl;
  const int n_pairs = (T + 1) * (T + 1), n_prow = tb.n_prow, n_pos = tb.n_pos;
  constexpr int D = TO_LABEL ? 0 : 1;
  const int rows = tb.rows[D];
  int *s_pair = reinterpret_cast<int *>(lsm);                          // [n_pairs][kPairInts]
  int *s_prow = s_pair + n_pairs * kPairInts;                          // [n_prow]
  int16_t *s_pos = reinterpret_cast<int16_t *>(s_prow + n_prow);       // [n_pos]
  float *s_coef = reinterpret_cast<float *>(s_prow + n_prow + (n_pos + 1) / 2);  // [rows][64]
  uint16_t *s_idx = reinterpret_cast<uint16_t *>(s_coef + 64 * rows);  // [rows][64]
  float *buf_all = lsm + lds_words(n_pairs, n_prow, n_pos, rows);      // [kLWaves][CB][n_lab]
  {
    const int *gp = reinterpret_cast<const int *>(tb.pair);
    for (int i = threadIdx.x; i < n_pairs * kPairInts; i += blockDim.x) s_pair[i] = gp[i];
    for (int i = threadIdx.x; i < n_prow; i += blockDim.x) s_prow[i] = tb.prow[i];
    for (int i = threadIdx.x; i < n_pos; i += blockDim.x) s_pos[i] = tb.pos[i];
    for (int i = threadIdx.x; i < 64 * rows; i += blockDim.x) {
      s_coef[i] = tb.coef[D][i];
      s_idx[i] = tb.idx[D][i];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x % kLW, wave = threadIdx.x / kLW;
  // staged inputs, then (once every pass has read them) the outputs, written out in order
  float *buf = buf_all + static_cast<size_t>(wave) * CB * n_lab;
  auto pinfo = [&](int pr) { return reinterpret_cast<const PairInfo *>(s_pair + pr * kPairInts); };
  // Rows are dealt to the XCDs in contiguous ranges (workgroup g runs on XCD
  // g % 8), so the rows of one structure, which read the same matrix lines,
  // share one L2.  Each wave walks its rows; rows without blocks are passed
  // over.  The blocks of a row are described 64 at a time (segment s0), one
  // block per lane.
  struct Pos {
    int64_t j;
    int e0, nb, s0;
  };
  const bool by_xcd = gridDim.x % 8 == 0;
  const int64_t xcd = blockIdx.x % 8, groups = by_xcd ? gridDim.x / 8 : gridDim.x;
  const int64_t local = by_xcd ? blockIdx.x / 8 : blockIdx.x;
  const int64_t j_end = by_xcd ? R.n_atoms * (xcd + 1) / 8 : R.n_atoms;
  const int64_t j_begin = by_xcd ? R.n_atoms * xcd / 8 : 0;
  const int64_t stride = groups * kLWaves;
  auto row_at = [&](int64_t j) {
    Pos p{j, 0, 0, 0};
    while (p.j < j_end) {
      int e1 = 0;
      if (!R.edges) {
        p.e0 = 0;
      } else if (!R.grouped) {
        p.e0 = R.row_ptr[p.j];
        e1 = R.row_ptr[p.j + 1];
      } else {  // a group's range, kept inside src_perm
        p.e0 = min(max(R.src_ptr[p.j], 0), R.n_edges);
        e1 = min(max(R.src_ptr[p.j + 1], p.e0), R.n_edges);
      }
      p.nb = R.nodes + (e1 - p.e0);
      if (p.nb > 0) break;
      p.j += stride;
    }
    return p;
  };
  auto next_seg = [&](Pos p) {
    p.s0 += kLW;
    return p.s0 < p.nb ? p : row_at(p.j + stride);
  };
  // lane l describes block s0 + l of the row (lanes past the row: empty)
  auto describe = [&](const Pos &p, unsigned long long *have) {
    Blk k{0, 0, 0, T * (T + 1) + T, R.nodes};
    const bool mine = p.j < j_end && p.s0 + lane < p.nb;
    bool ok = false;
    if (mine) k = block_of(R, tb, p.j, p.s0 + lane, p.e0, &ok);
    const unsigned long long bad = __ballot(mine && !ok);
    if (lane == 0 && bad && skipped) atomicAdd(skipped, static_cast<unsigned long long>(__popcll(bad)));
    *have = __ballot(mine);
    return k;
  };
  // A chunk: up to CB blocks of one template pair from one segment.
  struct Chunk {
    Blk k;             // the segment's descriptions (one block per lane)
    int lanes[CB];     // lanes of the chunk's blocks (repeats past nc)
    int nc, pair;
  };
  struct Cursor {
    Pos p;
    Blk k;
    unsigned long long rem, cm;  // lanes not yet taken; lanes of the current pair not yet taken
    int cp;
  };
  auto advance = [&](Cursor &c, Chunk &ch) {
    while (c.cm == 0 && c.rem == 0) {
      c.p = next_seg(c.p);
      if (c.p.j >= j_end) return false;
      c.k = describe(c.p, &c.rem);
    }
    if (c.cm == 0) {
      const int lead = __ffsll(c.rem) - 1;
      c.cp = __builtin_amdgcn_readlane(c.k.pair, lead);
      c.cm = __ballot(c.k.pair == c.cp) & c.rem;
      c.rem &= ~c.cm;
    }
    ch.k = c.k;
    ch.pair = c.cp;
    ch.nc = 0;
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      if (c.cm) {
        ch.lanes[b] = __ffsll(c.cm) - 1;
        c.cm &= c.cm - 1;
        ++ch.nc;
      } else {
        ch.lanes[b] = ch.lanes[0];
      }
    }
    return true;
  };
  auto rl = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
  auto rl64 = [](int64_t v, int l) {
    return (static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l)) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  };
  float v[NT][CB];
  // issue every load of a chunk before any of them is used; each block's
  // base is a wave-uniform pointer and its values 32-bit offsets from it
  auto issue = [&](const Chunk &ch) {
    const PairInfo &pi = *pinfo(ch.pair);
    const int P = pi.P;
    if constexpr (TO_LABEL) {
      // the pair's own entries p = lr * n_w + lc, one per lane and pass
      int lrs[NT], lcs[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int pe = lane + kLW * it;
        const int lr = (pe * pi.magic) >> 16;
        lrs[it] = pe < P ? lr : -1;
        lcs[it] = pe - lr * pi.n_w;
      }
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const float *bp = Hin + rl64(ch.k.base, ch.lanes[b]);
        const int ld = rl(ch.k.ld, ch.lanes[b]);
#pragma unroll
        for (int it = 0; it < NT; ++it) {
          // lanes past the pair's entries read the block's first entry (unused)
          const uint32_t off = lrs[it] >= 0 ? static_cast<uint32_t>(lrs[it] * ld + lcs[it]) : 0u;
          v[it][b] = bp[off];
        }
      }
    } else {
      // the labels the pair carries, in ascending label order (compact inputs i)
      int qs[NT];
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        const int i = lane + kLW * it;
        qs[it] = i < P ? s_pos[pi.spos + i] : 0;
      }
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const float *row = (rl(ch.k.node, ch.lanes[b]) ? lab_n_in : lab_e_in) + rl64(ch.k.out, ch.lanes[b]) * n_lab;
#pragma unroll
        for (int it = 0; it < NT; ++it) v[it][b] = row[static_cast<uint32_t>(qs[it])];
      }
    }
  };
  auto commit = [&](const Chunk &ch) {
    const int P = pinfo(ch.pair)->P;
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const int t = lane + kLW * it;
      if (t < P) {
#pragma unroll
        for (int b = 0; b < CB; ++b) buf[b * n_lab + t] = v[it][b];
      }
    }
  };
  auto outputs = [&](const Chunk &ch) {
    const PairInfo &pi = *pinfo(ch.pair);
    const int nc = ch.nc;
    if constexpr (TO_LABEL) {
      float *op[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b)
        op[b] = (rl(ch.k.node, ch.lanes[b]) ? lab_n_out : lab_e_out) + rl64(ch.k.out, ch.lanes[b]) * n_lab;
      // Eq. (1): the labels the pair carries, from their CG terms over the
      // staged entries (at most NT passes)
      float acc[NT][CB];
#pragma unroll
      for (int ps = 0; ps < NT; ++ps) {
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[ps][b] = 0.0f;
        if (ps < pi.lpass) {
          const int r1 = s_prow[pi.lprow + ps + 1];
          for (int rw = s_prow[pi.lprow + ps]; rw < r1; ++rw) {
            const float cf = s_coef[rw * 64 + lane];
            const int ix = s_idx[rw * 64 + lane];
#pragma unroll
            for (int b = 0; b < CB; ++b) acc[ps][b] += cf * buf[b * n_lab + ix];
          }
        }
      }
      wave_lds_order();
      // the output rows take the place of the staged entries
#pragma unroll
      for (int ps = 0; ps < NT; ++ps)
        if (ps < pi.lpass) {
          const int q = s_pos[pi.lpos + ps * 64 + lane];
          if (q >= 0) {
#pragma unroll
            for (int b = 0; b < CB; ++b) buf[b * n_lab + q] = acc[ps][b];
          }
        }
      // the labels of shell pairs the elements lack: the padding
      for (int ps = 0; ps < pi.zpass; ++ps) {
        const int q = s_pos[pi.zpos + ps * 64 + lane];
        if (q >= 0) {
#pragma unroll
          for (int b = 0; b < CB; ++b) buf[b * n_lab + q] = 0.0f;
        }
      }
      wave_lds_order();
      // whole rows out, 16 bytes per lane where the rows allow it
      if (R.vec4) {
        const int n4 = n_lab / 4;
#pragma unroll
        for (int b = 0; b < CB; ++b)
          if (b < nc)
            for (int c4 = lane; c4 < n4; c4 += kLW)
              reinterpret_cast<float4 *>(op[b])[c4] = reinterpret_cast<const float4 *>(buf + b * n_lab)[c4];
      } else {
#pragma unroll
        for (int b = 0; b < CB; ++b)
          if (b < nc)
            for (int q = lane; q < n_lab; q += kLW) op[b][q] = buf[b * n_lab + q];
      }
    } else {
      float *bp[CB];
      int ldb[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        bp[b] = Hout + rl64(ch.k.base, ch.lanes[b]);
        ldb[b] = rl(ch.k.ld, ch.lanes[b]);
      }
      // the pair's own entries from their CG terms over the staged labels
      // (at most NT passes), then in place of the staged labels
      float acc[NT][CB];
#pragma unroll
      for (int ps = 0; ps < NT; ++ps) {
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[ps][b] = 0.0f;
        if (ps < pi.epass) {
          const int r1 = s_prow[pi.eprow + ps + 1];
          for (int rw = s_prow[pi.eprow + ps]; rw < r1; ++rw) {
            const float cf = s_coef[rw * 64 + lane];
            const int ix = s_idx[rw * 64 + lane];
#pragma unroll
            for (int b = 0; b < CB; ++b) acc[ps][b] += cf * buf[b * n_lab + ix];
          }
        }
      }
      wave_lds_order();
#pragma unroll
      for (int ps = 0; ps < NT; ++ps)
        if (ps < pi.epass) {
          const int pe = s_pos[pi.epos + ps * 64 + lane];
          if (pe >= 0) {
#pragma unroll
            for (int b = 0; b < CB; ++b) buf[b * n_lab + pe] = acc[ps][b];
          }
        }
      wave_lds_order();
      // then out in row-major order: consecutive lanes write consecutive
      // columns of a block row
      const int P = pi.P;
      for (int pe = lane; pe < P; pe += kLW) {
        const int lr = (pe * pi.magic) >> 16, lc = pe - lr * pi.n_w;
#pragma unroll
        for (int b = 0; b < CB; ++b)
          if (b < nc) bp[b][static_cast<uint32_t>(lr * ldb[b] + lc)] = buf[b * n_lab + pe];
      }
    }
  };
  Cursor c;
  c.p = row_at(j_begin + local * kLWaves + wave);
  c.k = describe(c.p, &c.rem);
  c.cm = 0;
  c.cp = 0;
  Chunk cur, nxt;
  bool have = advance(c, cur);
  if (have) issue(cur);
  while (have) {
    commit(cur);
    wave_lds_order();
    // the next chunk's loads run while this chunk's outputs are formed
    const bool have_n = advance(c, nxt);
    if (have_n) issue(nxt);
    outputs(cur);
    wave_lds_order();
    cur = nxt;
    have = have_n;
  }
}

egnn_status check_orbitals(const egnn_orbitals *o, bool outputs) {
  EGNN_REQUIRE(o, "orbital layout is null");
  EGNN_REQUIRE(o->n_mols >= 0 && o->n_atoms >= 0, "negative structure or atom count");
  if (o->n_atoms > 0) EGNN_REQUIRE(o->species && o->atom_orb && o->atom_mol, "atom arrays are null");
  EGNN_REQUIRE(o->mol_ptr && o->mat_off, "structure arrays are null");
  if (o->n_mols > 0) EGNN_REQUIRE(o->mol_norb, "mol_norb is null");
  (void)outputs;
  return EGNN_OK;
}

egnn_status run_labels(bool to_label, const egnn_basis *b, const egnn_orbitals *o, const egnn_graph *g,
                       const float *Hin, float *Hout, int64_t h_elems, const float *le_in, const float *ln_in,
                       float *le_out, float *ln_out, int64_t *n_skipped, hipStream_t stream) {
  egnn_status st = check_orbitals(o, false);
  if (st != EGNN_OK) return st;
  const bool edges = g != nullptr && (to_label ? le_out != nullptr : le_in != nullptr);
  const bool nodes = to_label ? ln_out != nullptr : ln_in != nullptr;
  if (g) {
    EGNN_REQUIRE(g->n_dst == o->n_atoms && g->n_src == o->n_atoms,
                 "the graph's rows and sources must be the layout's atoms");
    EGNN_REQUIRE(g->n_edges >= 0, "negative edge count");
    EGNN_REQUIRE(g->n_edges <= INT_MAX, "more than 2^31 - 1 edges");
    if (edges) EGNN_REQUIRE(g->row_ptr && (g->n_edges == 0 || g->src), "graph arrays are null");
  }
  EGNN_REQUIRE(h_elems >= 0, "negative matrix size");
  const bool work = o->n_atoms > 0 && (edges || nodes);
  if (work) EGNN_REQUIRE(h_elems > 0 && (to_label ? Hin != nullptr : Hout != nullptr), "matrix storage is null or empty");
  int slot = 0;
  LInfo info{};
  st = label_slot(b, &slot, &info);
  if (st != EGNN_OK) return st;
  unsigned long long *skip = reinterpret_cast<unsigned long long *>(n_skipped);
  if (skip) {
    zero_u64<<<1, 1, 0, stream>>>(skip);
    EGNN_CHECK_LAUNCH();
  }
  if (!work) return EGNN_OK;
  // the source-grouped order when the graph carries it (one wave then owns a
  // source atom's row strip of the matrix: whole matrix rows for a fully
  // connected structure)
  const bool grouped = edges && g->src_ptr != nullptr && (g->n_edges == 0 || g->src_perm != nullptr);
  Rows R;
  R.n_atoms = o->n_atoms;
  R.n_mols = o->n_mols;
  R.row_ptr = edges ? g->row_ptr : nullptr;
  R.src = edges ? g->src : nullptr;
  R.shift = edges ? g->shift : nullptr;
  R.src_ptr = grouped ? g->src_ptr : nullptr;
  R.src_perm = grouped ? g->src_perm : nullptr;
  R.mol_ptr = o->mol_ptr;
  R.n_edges = edges ? static_cast<int>(g->n_edges) : 0;
  R.grouped = grouped ? 1 : 0;
  R.species = o->species;
  R.atom_orb = o->atom_orb;
  R.atom_mol = o->atom_mol;
  R.mol_norb = o->mol_norb;
  R.mat_off = o->mat_off;
  R.h_elems = h_elems;
  R.nodes = nodes ? 1 : 0;
  R.edges = edges ? 1 : 0;
  {
    auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    R.vec4 = info.n_lab % 4 == 0 && (!le_out || a16(le_out)) && (!ln_out || a16(ln_out)) ? 1 : 0;
  }
  const int n_rows = info.rows[to_label ? 0 : 1];
  const int64_t rows = (edges ? g->n_edges : 0) + (nodes ? o->n_atoms : 0);
  // algorithmic bytes when the graph covers every block once (a fully
  // connected structure): Matrix -> Label reads each matrix entry and writes
  // every label row; Label -> Matrix reads the labels the blocks carry (as
  // many as the matrix has entries) and writes each entry
  Timed tm(stream, to_label ? "matrix_to_label" : "label_to_matrix", 0.0,
           to_label ? 4.0 * (double(rows) * info.n_lab + double(h_elems)) : 8.0 * double(h_elems));
  if (grouped && g->n_edges > 0 && (skip || to_label)) {
    ungrouped_kernel<<<ceil_div(g->n_edges, 256), 256, 0, stream>>>(g->src, static_cast<int>(g->n_edges),
                                                                    o->n_atoms, info.n_lab,
                                                                    to_label ? le_out : nullptr, skip);
    EGNN_CHECK_LAUNCH();
  }
  // a multiple of 8 workgroups: rows are dealt to the XCDs in contiguous ranges
  int64_t blocks = ((static_cast<int64_t>(o->n_atoms) + kLWaves - 1) / kLWaves + 7) / 8 * 8;
  if (blocks > 2048) blocks = 2048;
  const size_t base_words = lds_words((info.n_tmpl + 1) * (info.n_tmpl + 1), info.n_prow, info.n_pos, n_rows);
  auto smem_for = [&](int cb) { return 4 * (base_words + static_cast<size_t>(kLWaves) * cb * info.n_lab); };
  auto launch = [&](auto cb, auto nt) -> egnn_status {
    constexpr int CB = decltype(cb)::value, NT = decltype(nt)::value;
    const size_t smem = smem_for(CB);
    if (to_label)
      labels_kernel<CB, NT, true><<<static_cast<unsigned>(blocks), kLW * kLWaves, smem, stream>>>(
          slot, R, Hin, nullptr, nullptr, nullptr, le_out, ln_out, skip);
    else
      labels_kernel<CB, NT, false><<<static_cast<unsigned>(blocks), kLW * kLWaves, smem, stream>>>(
          slot, R, nullptr, Hout, le_in, ln_in, nullptr, nullptr, skip);
    EGNN_CHECK_LAUNCH();
    return EGNN_OK;
  };
  // NT passes of 64 cover a block; CB blocks per chunk keep NT * CB values in
  // flight per lane.  CB is the largest whose staging fits in LDS, capped so
  // that the next chunk's values and this chunk's outputs fit in registers
  // (128 per lane at 16 waves): 4 up to 2 passes, 2 up to 12, 1 beyond.
  constexpr size_t kLds = 160 * 1024;
  const int passes = (info.n_lab + kLW - 1) / kLW;
  int cb = passes <= 2 ? 4 : passes <= 12 ? 2 : 1;
  while (cb > 1 && smem_for(cb) > kLds) cb /= 2;
  if (smem_for(cb) > kLds) {
    set_error("Matrix <-> Label needs %zu bytes of LDS; reduce the basis", smem_for(cb));
    return EGNN_E_UNSUPPORTED;
  }
  using std::integral_constant;
  auto with_cb = [&](auto nt) -> egnn_status {
    constexpr int NT = decltype(nt)::value;
    if (cb == 4 && NT <= 2) return launch(integral_constant<int, (NT <= 2 ? 4 : 1)>{}, nt);
    if (cb >= 2 && NT <= 12) return launch(integral_constant<int, (NT <= 12 ? 2 : 1)>{}, nt);
    return launch(integral_constant<int, 1>{}, nt);
  };
  if (passes <= 1) return with_cb(integral_constant<int, 1>{});
  if (passes <= 2) return with_cb(integral_constant<int, 2>{});
  if (passes <= 4) return with_cb(integral_constant<int, 4>{});
  if (passes <= 6) return with_cb(integral_constant<int, 6>{});
  if (passes <= 8) return with_cb(integral_constant<int, 8>{});
  if (passes <= 12) return with_cb(integral_constant<int, 12>{});
  return with_cb(integral_constant<int, 16>{});
}

}  // namespace
}  // namespace egnn

using namespace egnn;

extern "C" int32_t egnn_label_width(const egnn_basis *b) {
  std::vector<LabelTable> t(1);
  if (build_label_table(b, t.data())) return 0;
  return t[0].n_lab;
}

extern "C" egnn_status egnn_orbital_layout(const egnn_basis *b, egnn_orbitals *o, int64_t *n_invalid,
                                           hipStream_t stream) {
  clear_error();
  egnn_status st = check_orbitals(o, true);
  if (st != EGNN_OK) return st;
  int slot = 0;
  LInfo info{};
  st = label_slot(b, &slot, &info);
  if (st != EGNN_OK) return st;
  unsigned long long *bad = reinterpret_cast<unsigned long long *>(n_invalid);
  if (bad) {
    zero_u64<<<1, 1, 0, stream>>>(bad);
    EGNN_CHECK_LAUNCH();
  }
  Timed tm(stream, "orbital_layout", 0.0, 4.0 * (2.0 * o->n_atoms + 3.0 * o->n_mols) + 8.0 * o->n_mols);
  constexpr int T = 256;
  if (o->n_atoms > 0) {
    fill_i32<<<ceil_div(o->n_atoms, T), T, 0, stream>>>(o->atom_mol, o->n_atoms, -1);
    EGNN_CHECK_LAUNCH();
    fill_i32<<<ceil_div(o->n_atoms, T), T, 0, stream>>>(o->atom_orb, o->n_atoms, 0);
    EGNN_CHECK_LAUNCH();
  }
  if (o->n_mols > 0) {
    int64_t blocks = (static_cast<int64_t>(o->n_mols) * kLW + T - 1) / T;
    if (blocks > 4096) blocks = 4096;
    layout_kernel<<<static_cast<unsigned>(blocks), T, 0, stream>>>(slot, o->n_mols, o->n_atoms, o->mol_ptr,
                                                                   o->species, o->atom_orb, o->atom_mol,
                                                                   o->mol_norb, bad);
    EGNN_CHECK_LAUNCH();
  }
  mat_off_kernel<<<1, 1024, 0, stream>>>(o->n_mols, o->mol_norb, o->mat_off);
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}

extern "C" egnn_status egnn_matrix_to_label(const egnn_basis *b, const egnn_orbitals *o, const egnn_graph *g,
                                            const float *H, int64_t h_elems, float *h_edge, float *h_node,
                                            int64_t *n_skipped, hipStream_t stream) {
  clear_error();
  return run_labels(true, b, o, g, H, nullptr, h_elems, nullptr, nullptr, h_edge, h_node, n_skipped, stream);
}

extern "C" egnn_status egnn_label_to_matrix(const egnn_basis *b, const egnn_orbitals *o, const egnn_graph *g,
                                            const float *h_edge, const float *h_node, float *H, int64_t h_elems,
                                            int64_t *n_skipped, hipStream_t stream) {
  clear_error();
  return run_labels(false, b, o, g, nullptr, H, h_elems, h_edge, h_node, nullptr, nullptr, n_skipped, stream);
}
