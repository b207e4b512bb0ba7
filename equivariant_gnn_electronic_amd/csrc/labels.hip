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
// block per node or edge.  Here one 64-lane wave owns a destination row.  It
// takes the row's on-site block and its edges CB at a time and stages them
// in LDS in the full shape, with lanes over entries and CB independent loads
// per lane in flight.  Lanes then run over labels (or entries) and sum the
// sparse CG terms of each from an LDS copy of the table; each term is read
// once for all CB blocks.
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
constexpr int kEntMax = kFullMax * kFullMax;
constexpr int kPassMax = kEntMax / 64;       // 64-lane passes over a block's labels or entries
constexpr int kRowMax = 256;                 // padded term rows of one direction
constexpr int kSpeciesMax = 64;
constexpr int kShellLMax = 3;                // s, p, d, f shells: labels up to L = 6

// One direction of the transform (labels from entries, or entries from
// labels) in lane-major form: the outputs are ordered by their number of CG
// terms (most first) and dealt to the lanes of 64-wide passes; pass p reads
// padded term rows prow[p] .. prow[p+1]-1, lane l taking coef / idx
// [row][l] (zero coefficients pad the shorter lists), so every lane of a
// pass runs the same number of terms and the reads are lane-contiguous.
struct LDir {
  int n_pass;
  int prow[kPassMax + 1];
  int16_t pos[kPassMax * 64];                // output of each lane of each pass, -1 if none
  float coef[kRowMax * 64];
  uint16_t idx[kRowMax * 64];                // input of each term (entry r * n_full + c, or label q)
};

struct LabelTable {
  int n_full, n_lab, n_species;
  int n_orb[kSpeciesMax + 1];                // the last row stands for an index outside the table
  int8_t omap[kSpeciesMax + 1][kFullMax];    // own orbital of each full orbital, -1 if absent
  LDir to_lab;                               // Matrix -> Label: label q from block entries
  LDir to_ent;                               // Label -> Matrix: entry t from labels
};

__device__ LabelTable g_ltables[kLSlots];

// Builds the table; returns nullptr, or why the basis is not accepted.
const char *build_label_table(const egnn_basis *b, LabelTable *t) {
  if (!b || !b->shell_l || !b->species_shells) return "basis pointers are null";
  if (b->n_shells < 1 || b->n_shells > 16) return "n_shells must be 1..16";
  if (b->n_species < 1 || b->n_species > kSpeciesMax) return "n_species must be 1..64";
  std::vector<int> off(b->n_shells);
  int o = 0, lmx = 0;
  for (int a = 0; a < b->n_shells; ++a) {
    const int l = b->shell_l[a];
    if (l < 0 || l > kShellLMax) return "shell degrees must be 0..3";
    off[a] = o;
    o += 2 * l + 1;
    lmx = std::max(lmx, l);
  }
  if (o > kFullMax) return "the full shell list has more than 32 orbitals";
  for (int z = 0; z < b->n_species; ++z)
    if (b->species_shells[z] >> b->n_shells) return "a species mask names a shell beyond n_shells";
  std::memset(t, 0, sizeof(*t));
  std::memset(t->omap, 0xFF, sizeof(t->omap));
  t->n_full = o;
  t->n_lab = o * o;
  t->n_species = b->n_species;
  for (int z = 0; z < b->n_species; ++z) {
    int oo = 0;
    for (int a = 0; a < b->n_shells; ++a)
      if ((b->species_shells[z] >> a) & 1u) {
        const int l = b->shell_l[a];
        for (int m = 0; m < 2 * l + 1; ++m) t->omap[z][off[a] + m] = static_cast<int8_t>(oo + m);
        oo += 2 * l + 1;
      }
    t->n_orb[z] = oo;
  }
  // label channels: ordered shell pairs in lexicographic order, L ascending
  const int Lmax = 2 * lmx;
  std::vector<int> nL(Lmax + 1, 0), hoff(Lmax + 2, 0);
  struct Item { int a, b, L, k; };
  std::vector<Item> items;
  for (int a = 0; a < b->n_shells; ++a)
    for (int c = 0; c < b->n_shells; ++c)
      for (int L = std::abs(b->shell_l[a] - b->shell_l[c]); L <= b->shell_l[a] + b->shell_l[c]; ++L)
        items.push_back({a, c, L, nL[L]++});
  for (int L = 0; L <= Lmax; ++L) hoff[L + 1] = hoff[L] + (2 * L + 1) * nL[L];
  if (hoff[Lmax + 1] != o * o) return "internal: label count differs from the block size";
  std::vector<std::vector<std::pair<float, int>>> by_lab(o * o), by_ent(o * o);
  for (const Item &it : items) {
    const int la = b->shell_l[it.a], lb = b->shell_l[it.b];
    const std::vector<double> Q = cg::real_coupling(la, lb, it.L);
    const int nb = 2 * lb + 1, nm = 2 * it.L + 1;
    for (int i = 0; i < 2 * la + 1; ++i)
      for (int j = 0; j < nb; ++j)
        for (int M = 0; M < nm; ++M) {
          const double c = Q[(i * nb + j) * nm + M];
          if (std::fabs(c) < 1e-12) continue;
          const int ent = (off[it.a] + i) * o + off[it.b] + j;
          const int q = hoff[it.L] + M * nL[it.L] + it.k;
          by_lab[q].push_back({static_cast<float>(c), ent});
          by_ent[ent].push_back({static_cast<float>(c), q});
        }
  }
  auto deal = [&](const std::vector<std::vector<std::pair<float, int>>> &v, LDir *d) {
    const int n = static_cast<int>(v.size());
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int c) { return v[a].size() > v[c].size(); });
    d->n_pass = (n + 63) / 64;
    int row = 0;
    for (int p = 0; p < d->n_pass; ++p) {
      size_t iters = 0;
      for (int l = 0; l < 64; ++l) {
        const int k = p * 64 + l;
        d->pos[k] = static_cast<int16_t>(k < n ? order[k] : -1);
        if (k < n) iters = std::max(iters, v[order[k]].size());
      }
      d->prow[p] = row;
      if (row + static_cast<int>(iters) > kRowMax) return false;
      for (size_t it = 0; it < iters; ++it, ++row)
        for (int l = 0; l < 64; ++l) {
          const int k = p * 64 + l;
          const bool has = k < n && it < v[order[k]].size();
          d->coef[row * 64 + l] = has ? v[order[k]][it].first : 0.0f;
          d->idx[row * 64 + l] = static_cast<uint16_t>(has ? v[order[k]][it].second : 0);
        }
    }
    d->prow[d->n_pass] = row;
    return true;
  };
  if (!deal(by_lab, &t->to_lab) || !deal(by_ent, &t->to_ent)) return "too many coupling terms for the table";
  return nullptr;
}

struct LKey {
  int n_shells, n_species;
  int l[16];
  uint32_t mask[kSpeciesMax];
};
struct LInfo {
  int n_full, n_lab, n_species, lab_rows, ent_rows, n_pass;
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
  in.lab_rows = t[0].to_lab.prow[t[0].to_lab.n_pass];
  in.ent_rows = t[0].to_ent.prow[t[0].to_ent.n_pass];
  in.n_pass = t[0].to_lab.n_pass;
  g_lcache.used[dev] = s + 1;
  *slot = s;
  *info = in;
  return EGNN_OK;
}

constexpr int kLW = 64;
constexpr int kLWaves = 4;

__global__ void fill_i32(int *p, int64_t n, int v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void zero_u64(unsigned long long *p) { *p = 0ull; }

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
  const int *species, *atom_orb, *atom_mol, *mol_norb;
  const int64_t *mat_off;
  int64_t h_elems;
  int nodes, edges;  // 1 = on-site blocks / edge blocks requested
};

// Block bi of destination row j: the on-site block first (when requested),
// then the row's edges.  ok = 0 when the block has no place in a matrix.
struct Blk {
  int64_t base, out;
  int ld, zi, zj, ok, node;
};

__device__ inline Blk block_of(const Rows &R, int n_species, const int *norb, int64_t j, int bi, int e0) {
  Blk k;
  int i;
  if (R.nodes && bi == 0) {
    i = static_cast<int>(j);
    k.node = 1;
    k.out = j;
  } else {
    const int64_t e = static_cast<int64_t>(e0) + bi - R.nodes;
    i = R.src[e];
    k.node = 0;
    k.out = e;
  }
  bool ok = i >= 0 && i < R.n_atoms;
  if (!k.node && R.shift) {
    const int8_t *s = R.shift + 3 * k.out;
    ok = ok && s[0] == 0 && s[1] == 0 && s[2] == 0;
  }
  const int ic = ok ? i : 0;
  const int mj = R.atom_mol[j], mi = R.atom_mol[ic];
  ok = ok && mj >= 0 && mj < R.n_mols && mi == mj;
  const int si = R.species[ic], sj = R.species[j];
  k.zi = (si >= 0 && si < n_species) ? si : n_species;
  k.zj = (sj >= 0 && sj < n_species) ? sj : n_species;
  int ld = 0;
  int64_t mo = 0;
  if (ok) {  // only then is mj a structure (there may be none)
    ld = R.mol_norb[mj];
    mo = R.mat_off[mj];
  }
  const int oi = R.atom_orb[ic], oj = R.atom_orb[j];
  // (ld < 2^26 keeps the 32-bit entry offsets r * ld + c of the kernels exact)
  ok = ok && ld >= 0 && ld < (1 << 26) && oi >= 0 && oj >= 0 && oi + norb[k.zi] <= ld && oj + norb[k.zj] <= ld && mo >= 0 &&
       mo + static_cast<int64_t>(ld) * ld <= R.h_elems;
  k.ok = ok;
  k.ld = ok ? ld : 0;
  k.base = ok ? mo + static_cast<int64_t>(oi) * ld + oj : 0;
  return k;
}

// LDS: one direction's passes (prow, pos, coef, idx), templates (omap,
// n_orb), then per wave CB staged blocks.
__host__ __device__ inline size_t lds_words(int n_pass, int rows, int n_species, int n_full) {
  return (static_cast<size_t>(n_pass + 1) + 64 * static_cast<size_t>(n_pass) + 128 * static_cast<size_t>(rows) +
          static_cast<size_t>(n_species + 1) * (n_full + 1) + 3) & ~static_cast<size_t>(3);
}

template <int CB, int NT, bool TO_LABEL>
__global__ void __launch_bounds__(kLW * kLWaves) labels_kernel(int slot, Rows R, const float *__restrict__ Hin,
                                                                float *__restrict__ Hout,
                                                                const float *__restrict__ lab_e_in,
                                                                const float *__restrict__ lab_n_in,
                                                                float *__restrict__ lab_e_out,
                                                                float *__restrict__ lab_n_out,
                                                                unsigned long long *skipped) {
  static_assert(NT * CB <= 64, "one presence bit per staged value");
  extern __shared__ float lsm[];
  const LabelTable &tb = g_ltables[slot];
  const int nf = tb.n_full, n_lab = tb.n_lab, nsp = tb.n_species;
  const LDir &dir = TO_LABEL ? tb.to_lab : tb.to_ent;
  const int n_pass = dir.n_pass, n_rows = dir.prow[n_pass];
  int *s_prow = reinterpret_cast<int *>(lsm);                      // [n_pass + 1]
  int *s_pos = s_prow + (n_pass + 1);                              // [n_pass][64]
  float *s_coef = reinterpret_cast<float *>(s_pos + 64 * n_pass);  // [n_rows][64]
  int *s_idx = reinterpret_cast<int *>(s_coef + 64 * n_rows);      // [n_rows][64]
  int *omap = s_idx + 64 * n_rows;                                 // [nsp + 1][nf]
  int *norb = omap + (nsp + 1) * nf;                               // [nsp + 1]
  float *buf_all = lsm + lds_words(n_pass, n_rows, nsp, nf);       // [kLWaves][CB][n_lab]
  for (int i = threadIdx.x; i <= n_pass; i += blockDim.x) s_prow[i] = dir.prow[i];
  for (int i = threadIdx.x; i < 64 * n_pass; i += blockDim.x) s_pos[i] = dir.pos[i];
  for (int i = threadIdx.x; i < 64 * n_rows; i += blockDim.x) {
    s_coef[i] = dir.coef[i];
    s_idx[i] = dir.idx[i];
  }
  for (int i = threadIdx.x; i < (nsp + 1) * nf; i += blockDim.x) {
    const int z = i / nf;
    omap[i] = tb.omap[z == nsp ? kSpeciesMax : z][i - z * nf];
  }
  for (int i = threadIdx.x; i <= nsp; i += blockDim.x) norb[i] = i == nsp ? 0 : tb.n_orb[i];
  __syncthreads();
  const int lane = threadIdx.x % kLW, wave = threadIdx.x / kLW;
  float *buf = buf_all + static_cast<size_t>(wave) * CB * n_lab;
  // the entries (r, c) this lane stages, one per pass over the block
  // (clamped to entry 0 past the block; `tin` bit it says the entry exists)
  int rr[NT], cc[NT];
  uint32_t tin = 0;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    const int t = lane + kLW * it;
    const bool in = t < n_lab;
    rr[it] = in ? t / nf : 0;
    cc[it] = in ? t - (t / nf) * nf : 0;
    tin |= static_cast<uint32_t>(in) << it;
  }
  // Label -> Matrix: the entry (er, ec) each lane forms in each pass (-1: none)
  int er[NT], ec[NT];
#pragma unroll
  for (int ps = 0; ps < NT; ++ps) {
    const int t = ps < n_pass ? s_pos[ps * 64 + lane] : -1;
    er[ps] = t >= 0 ? t / nf : -1;
    ec[ps] = t >= 0 ? t - er[ps] * nf : 0;
  }
  (void)er;
  (void)ec;
  // Rows are dealt to the XCDs in contiguous ranges (workgroup g runs on XCD
  // g % 8), so the rows of one structure, which read the same matrix lines,
  // share one L2.  Each wave's chunks form one sequence (row j, first block
  // c0); rows without blocks are passed over.  The blocks of a row are
  // described 64 at a time (segment s0), one block per lane.
  struct Pos {
    int64_t j;
    int e0, nb, s0, c0;
  };
  const bool by_xcd = gridDim.x % 8 == 0;
  const int64_t xcd = blockIdx.x % 8, groups = by_xcd ? gridDim.x / 8 : gridDim.x;
  const int64_t local = by_xcd ? blockIdx.x / 8 : blockIdx.x;
  const int64_t j_end = by_xcd ? R.n_atoms * (xcd + 1) / 8 : R.n_atoms;
  const int64_t j_begin = by_xcd ? R.n_atoms * xcd / 8 : 0;
  const int64_t stride = groups * kLWaves;
  auto row_at = [&](int64_t j) {
    Pos p{j, 0, 0, 0, 0};
    while (p.j < j_end) {
      p.e0 = R.edges ? R.row_ptr[p.j] : 0;
      p.nb = R.nodes + (R.edges ? R.row_ptr[p.j + 1] - p.e0 : 0);
      if (p.nb > 0) break;
      p.j += stride;
    }
    return p;
  };
  auto next = [&](Pos p) {
    p.c0 += CB;
    if (p.c0 >= p.nb) return row_at(p.j + stride);
    if (p.c0 >= p.s0 + kLW) p.s0 += kLW;
    return p;
  };
  // lane l describes block s0 + l of the row (blocks past the row are empty
  // slots pointing at row 0 of a kind of block that exists: the on-site rows
  // whenever they are requested, else the first edge)
  auto describe = [&](const Pos &p) {
    Blk k{0, 0, 0, nsp, nsp, 0, R.nodes};
    const bool mine = p.j < j_end && p.s0 + lane < p.nb;
    if (mine) k = block_of(R, nsp, norb, p.j, p.s0 + lane, p.e0);
    const unsigned long long bad = __ballot(mine && !k.ok);
    if (lane == 0 && bad && skipped) atomicAdd(skipped, static_cast<unsigned long long>(__popcll(bad)));
    return k;
  };
  auto rl = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };
  auto rl64 = [](int64_t v, int l) {
    return (static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l)) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  };
  float v[NT][CB];
  using Mask = typename std::conditional<(NT * CB <= 32), uint32_t, unsigned long long>::type;
  Mask pres = 0;  // bit it * CB + b: value v[it][b] is a matrix entry (Matrix -> Label)
  // issue every load of a chunk before any of them is used; each block's
  // base is a wave-uniform pointer and the entries 32-bit offsets from it
  auto issue = [&](const Blk &k, const Pos &p) {
    const int l0 = p.c0 - p.s0;
    if constexpr (TO_LABEL) {
      pres = 0;
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const float *bp = Hin + rl64(k.base, l0 + b);
        const int ld = rl(k.ld, l0 + b), oi = rl(k.zi, l0 + b) * nf, oj = rl(k.zj, l0 + b) * nf;
        const bool ok = rl(k.ok, l0 + b) != 0;
#pragma unroll
        for (int it = 0; it < NT; ++it) {
          const int lr = omap[oi + rr[it]], lc = omap[oj + cc[it]];
          const bool pr = ok & ((tin >> it) & 1u) & (lr >= 0) & (lc >= 0);
          // absent entries read the block's first element (element 0 of H for
          // a block with no place) and are zeroed when staged
          const uint32_t off = pr ? static_cast<uint32_t>(lr * ld + lc) : 0u;
          v[it][b] = bp[off];
          pres |= static_cast<Mask>(pr) << (it * CB + b);
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const float *row = (rl(k.node, l0 + b) ? lab_n_in : lab_e_in) + rl64(k.out, l0 + b) * n_lab;
#pragma unroll
        for (int it = 0; it < NT; ++it) v[it][b] = row[static_cast<uint32_t>(min(lane + kLW * it, n_lab - 1))];
      }
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      const int t = lane + kLW * it;
      if (t < n_lab) {
#pragma unroll
        for (int b = 0; b < CB; ++b) {
          float x = v[it][b];
          if constexpr (TO_LABEL) x = ((pres >> (it * CB + b)) & 1u) ? x : 0.0f;
          buf[b * n_lab + t] = x;
        }
      }
    }
  };
  Pos p = row_at(j_begin + local * kLWaves + wave);
  Blk k = describe(p);
  if (p.j < j_end) issue(k, p);
  while (p.j < j_end) {
    const int nc = min(CB, p.nb - p.c0);
    const int l0 = p.c0 - p.s0;
    commit();
    wave_lds_order();
    // the next chunk's loads run while this chunk's outputs are formed
    const Pos pn = next(p);
    const Blk kn = (pn.j != p.j || pn.s0 != p.s0) ? describe(pn) : k;
    if (pn.j < j_end) issue(kn, pn);
    if constexpr (TO_LABEL) {
      // Eq. (1): the labels of each block from their CG terms over the staged
      // entries, one pass of 64 labels at a time
      float *op[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b)
        op[b] = (rl(k.node, l0 + b) ? lab_n_out : lab_e_out) + rl64(k.out, l0 + b) * n_lab;
      for (int ps = 0; ps < n_pass; ++ps) {
        float acc[CB];
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[b] = 0.0f;
        const int r1 = s_prow[ps + 1];
        for (int rw = s_prow[ps]; rw < r1; ++rw) {
          const float cf = s_coef[rw * 64 + lane];
          const int ix = s_idx[rw * 64 + lane];
#pragma unroll
          for (int b = 0; b < CB; ++b) acc[b] += cf * buf[b * n_lab + ix];
        }
        const int q = s_pos[ps * 64 + lane];
        if (q >= 0) {
#pragma unroll
          for (int b = 0; b < CB; ++b)
            if (b < nc) op[b][static_cast<uint32_t>(q)] = acc[b];
        }
      }
    } else {
      // entries from their CG terms over the staged labels, written where the
      // template has an orbital
      float *bp[CB];
      int ldb[CB], oib[CB], ojb[CB];
      bool okb[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        bp[b] = Hout + rl64(k.base, l0 + b);
        ldb[b] = rl(k.ld, l0 + b);
        oib[b] = rl(k.zi, l0 + b) * nf;
        ojb[b] = rl(k.zj, l0 + b) * nf;
        okb[b] = b < nc && rl(k.ok, l0 + b) != 0;
      }
#pragma unroll
      for (int ps = 0; ps < NT; ++ps) {
        if (ps >= n_pass) break;
        float acc[CB];
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[b] = 0.0f;
        const int r1 = s_prow[ps + 1];
        for (int rw = s_prow[ps]; rw < r1; ++rw) {
          const float cf = s_coef[rw * 64 + lane];
          const int ix = s_idx[rw * 64 + lane];
#pragma unroll
          for (int b = 0; b < CB; ++b) acc[b] += cf * buf[b * n_lab + ix];
        }
        if (er[ps] >= 0) {
#pragma unroll
          for (int b = 0; b < CB; ++b) {
            const int lr = omap[oib[b] + er[ps]], lc = omap[ojb[b] + ec[ps]];
            if (okb[b] && lr >= 0 && lc >= 0) bp[b][static_cast<uint32_t>(lr * ldb[b] + lc)] = acc[b];
          }
        }
      }
    }
    wave_lds_order();
    p = pn;
    k = kn;
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
  Rows R;
  R.n_atoms = o->n_atoms;
  R.n_mols = o->n_mols;
  R.row_ptr = edges ? g->row_ptr : nullptr;
  R.src = edges ? g->src : nullptr;
  R.shift = edges ? g->shift : nullptr;
  R.species = o->species;
  R.atom_orb = o->atom_orb;
  R.atom_mol = o->atom_mol;
  R.mol_norb = o->mol_norb;
  R.mat_off = o->mat_off;
  R.h_elems = h_elems;
  R.nodes = nodes ? 1 : 0;
  R.edges = edges ? 1 : 0;
  const int n_rows = to_label ? info.lab_rows : info.ent_rows;
  const int64_t rows = (edges ? g->n_edges : 0) + (nodes ? o->n_atoms : 0);
  // algorithmic bytes: every label row once, and every matrix entry once
  // when the graph covers each block (a fully connected structure)
  Timed tm(stream, to_label ? "matrix_to_label" : "label_to_matrix", 0.0,
           4.0 * (double(rows) * info.n_lab + double(h_elems)));
  // a multiple of 8 workgroups: rows are dealt to the XCDs in contiguous ranges
  int64_t blocks = ((static_cast<int64_t>(o->n_atoms) + kLWaves - 1) / kLWaves + 7) / 8 * 8;
  if (blocks > 2048) blocks = 2048;
  const size_t base_words = lds_words(info.n_pass, n_rows, info.n_species, info.n_full);
  auto launch = [&](auto cb, auto nt) -> egnn_status {
    constexpr int CB = decltype(cb)::value, NT = decltype(nt)::value;
    const size_t smem = 4 * (base_words + static_cast<size_t>(kLWaves) * CB * info.n_lab);
    if (smem > 160 * 1024) {
      set_error("Matrix <-> Label needs %zu bytes of LDS; reduce the basis", smem);
      return EGNN_E_UNSUPPORTED;
    }
    if (to_label)
      labels_kernel<CB, NT, true><<<static_cast<unsigned>(blocks), kLW * kLWaves, smem, stream>>>(
          slot, R, Hin, nullptr, nullptr, nullptr, le_out, ln_out, skip);
    else
      labels_kernel<CB, NT, false><<<static_cast<unsigned>(blocks), kLW * kLWaves, smem, stream>>>(
          slot, R, nullptr, Hout, le_in, ln_in, nullptr, nullptr, skip);
    EGNN_CHECK_LAUNCH();
    return EGNN_OK;
  };
  // NT passes of 64 entries cover a block; CB blocks per chunk keep NT * CB
  // values in flight per lane
  const int passes = (info.n_lab + kLW - 1) / kLW;
  if (passes <= 1) return launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 1>{});
  if (passes <= 2) return launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 2>{});
  if (passes <= 4) return launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 4>{});
  if (passes <= 6) return launch(std::integral_constant<int, 4>{}, std::integral_constant<int, 6>{});
  if (passes <= 8) return launch(std::integral_constant<int, 4>{}, std::integral_constant<int, 8>{});
  if (passes <= 12) return launch(std::integral_constant<int, 2>{}, std::integral_constant<int, 12>{});
  return launch(std::integral_constant<int, 2>{}, std::integral_constant<int, 16>{});
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
