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
#include <climits>
#include <cstring>
#include <mutex>
#include <vector>

#include "cg_real.h"
#include "common.h"
#include "timing.h"

namespace egnn {
namespace {

constexpr int kLSlots = 4;
constexpr int kFullMax = 32;                 // orbitals of the full shell list
constexpr int kEntMax = kFullMax * kFullMax;
constexpr int kTermMax = 8192;
constexpr int kSpeciesMax = 64;
constexpr int kShellLMax = 3;                // s, p, d, f shells: labels up to L = 6

struct LabelTable {
  int n_full, n_lab, n_species;
  int n_orb[kSpeciesMax + 1];                // the last row stands for an index outside the table
  int8_t omap[kSpeciesMax + 1][kFullMax];    // own orbital of each full orbital, -1 if absent
  int lab_start[kEntMax + 1];                // Matrix -> Label: terms of label q ...
  float lab_coef[kTermMax];
  uint16_t lab_ent[kTermMax];                // ... over block entries r * n_full + c
  int ent_start[kEntMax + 1];                // Label -> Matrix: terms of entry t ...
  float ent_coef[kTermMax];
  uint16_t ent_lab[kTermMax];                // ... over labels
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
  auto flatten = [&](const std::vector<std::vector<std::pair<float, int>>> &v, int *start, float *coef,
                     uint16_t *idx) {
    int n = 0;
    for (size_t r = 0; r < v.size(); ++r) {
      start[r] = n;
      for (const auto &p : v[r]) {
        if (n >= kTermMax) return false;
        coef[n] = p.first;
        idx[n] = static_cast<uint16_t>(p.second);
        ++n;
      }
    }
    start[v.size()] = n;
    return true;
  };
  if (!flatten(by_lab, t->lab_start, t->lab_coef, t->lab_ent) ||
      !flatten(by_ent, t->ent_start, t->ent_coef, t->ent_lab))
    return "too many coupling terms for the table";
  return nullptr;
}

struct LKey {
  int n_shells, n_species;
  int l[16];
  uint32_t mask[kSpeciesMax];
};
struct LInfo {
  int n_full, n_lab, n_species, lab_terms, ent_terms;
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
  in.lab_terms = t[0].lab_start[in.n_lab];
  in.ent_terms = t[0].ent_start[in.n_lab];
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
  ok = ok && ld >= 0 && oi >= 0 && oj >= 0 && oi + norb[k.zi] <= ld && oj + norb[k.zj] <= ld && mo >= 0 &&
       mo + static_cast<int64_t>(ld) * ld <= R.h_elems;
  k.ok = ok;
  k.ld = ok ? ld : 0;
  k.base = ok ? mo + static_cast<int64_t>(oi) * ld + oj : 0;
  return k;
}

// LDS: term table (start, coef, index), templates (omap, n_orb), then per wave CB label buffers.
__host__ __device__ inline size_t lds_words(int n_lab, int n_terms, int n_species, int n_full) {
  return (static_cast<size_t>(n_lab + 1) + 2 * n_terms + static_cast<size_t>(n_species + 1) * (n_full + 1) + 3) & ~3;
}

template <int CB, bool TO_LABEL>
__global__ void __launch_bounds__(kLW * kLWaves) labels_kernel(int slot, Rows R, const float *__restrict__ Hin,
                                                                float *__restrict__ Hout,
                                                                const float *__restrict__ lab_e_in,
                                                                const float *__restrict__ lab_n_in,
                                                                float *__restrict__ lab_e_out,
                                                                float *__restrict__ lab_n_out,
                                                                unsigned long long *skipped) {
  extern __shared__ float lsm[];
  const LabelTable &tb = g_ltables[slot];
  const int nf = tb.n_full, n_lab = tb.n_lab, nsp = tb.n_species;
  const int *g_start = TO_LABEL ? tb.lab_start : tb.ent_start;
  const float *g_coef = TO_LABEL ? tb.lab_coef : tb.ent_coef;
  const uint16_t *g_idx = TO_LABEL ? tb.lab_ent : tb.ent_lab;
  const int n_terms = g_start[n_lab];
  int *t_start = reinterpret_cast<int *>(lsm);                     // [n_lab + 1]
  float *t_coef = lsm + (n_lab + 1);                               // [n_terms]
  int *t_idx = reinterpret_cast<int *>(t_coef + n_terms);          // [n_terms]
  int *omap = t_idx + n_terms;                                     // [nsp + 1][nf]
  int *norb = omap + (nsp + 1) * nf;                               // [nsp + 1]
  float *buf_all = lsm + lds_words(n_lab, n_terms, nsp, nf);       // [kLWaves][CB][n_lab]
  for (int i = threadIdx.x; i <= n_lab; i += blockDim.x) t_start[i] = g_start[i];
  for (int i = threadIdx.x; i < n_terms; i += blockDim.x) {
    t_coef[i] = g_coef[i];
    t_idx[i] = g_idx[i];
  }
  for (int i = threadIdx.x; i < (nsp + 1) * nf; i += blockDim.x) {
    const int z = i / nf;
    omap[i] = tb.omap[z == nsp ? kSpeciesMax : z][i - z * nf];
  }
  for (int i = threadIdx.x; i <= nsp; i += blockDim.x) norb[i] = i == nsp ? 0 : tb.n_orb[i];
  __syncthreads();
  const int lane = threadIdx.x % kLW, wave = threadIdx.x / kLW;
  float *buf = buf_all + static_cast<size_t>(wave) * CB * n_lab;
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * kLWaves + wave; j < R.n_atoms;
       j += static_cast<int64_t>(gridDim.x) * kLWaves) {
    const int e0 = R.edges ? R.row_ptr[j] : 0;
    const int nb = R.nodes + (R.edges ? R.row_ptr[j + 1] - e0 : 0);
    for (int c0 = 0; c0 < nb; c0 += CB) {
      const int nc = min(CB, nb - c0);
      // lane b < nc describes block c0 + b; the wave reads the descriptions
      // back as scalars
      Blk mine{0, 0, 0, nsp, nsp, 0, 0};
      if (lane < nc) mine = block_of(R, nsp, norb, j, c0 + lane, e0);
      const unsigned long long bad = __ballot(lane < nc && !mine.ok);
      if (lane == 0 && bad && skipped) atomicAdd(skipped, static_cast<unsigned long long>(__popcll(bad)));
      int64_t base[CB], out[CB];
      int ld[CB], zi[CB], zj[CB], ok[CB], node[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        base[b] = (static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(mine.base >> 32), b)) << 32) |
                  static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine.base), b));
        out[b] = (static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(mine.out >> 32), b)) << 32) |
                 static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine.out), b));
        ld[b] = __builtin_amdgcn_readlane(mine.ld, b);
        zi[b] = __builtin_amdgcn_readlane(mine.zi, b);
        zj[b] = __builtin_amdgcn_readlane(mine.zj, b);
        ok[b] = __builtin_amdgcn_readlane(mine.ok, b);
        node[b] = __builtin_amdgcn_readlane(mine.node, b);
      }
      if constexpr (TO_LABEL) {
        // (1) extract: entry t = (r, c) of the full shape, zero where the
        // template has no orbital (clamped loads, then a select: no branch
        // between the CB loads)
        for (int t = lane; t < n_lab; t += kLW) {
          const int r = t / nf, c = t - r * nf;
          float v[CB];
          bool p[CB];
#pragma unroll
          for (int b = 0; b < CB; ++b) {
            const int lr = omap[zi[b] * nf + r], lc = omap[zj[b] * nf + c];
            p[b] = b < nc && ok[b] && lr >= 0 && lc >= 0;
            v[b] = Hin[p[b] ? base[b] + static_cast<int64_t>(lr) * ld[b] + lc : 0];
          }
#pragma unroll
          for (int b = 0; b < CB; ++b) buf[b * n_lab + t] = p[b] ? v[b] : 0.0f;
        }
        wave_lds_order();
        // (2) Eq. (1): label q of each block from its CG terms
        for (int q = lane; q < n_lab; q += kLW) {
          float acc[CB];
#pragma unroll
          for (int b = 0; b < CB; ++b) acc[b] = 0.0f;
          const int t1 = t_start[q + 1];
          for (int k = t_start[q]; k < t1; ++k) {
            const float cf = t_coef[k];
            const int ix = t_idx[k];
#pragma unroll
            for (int b = 0; b < CB; ++b) acc[b] += cf * buf[b * n_lab + ix];
          }
#pragma unroll
          for (int b = 0; b < CB; ++b)
            if (b < nc) (node[b] ? lab_n_out : lab_e_out)[out[b] * n_lab + q] = acc[b];
        }
        wave_lds_order();
      } else {
        // labels of the CB blocks into LDS (rows of n_lab floats)
        for (int q = lane; q < n_lab; q += kLW) {
          float v[CB];
#pragma unroll
          for (int b = 0; b < CB; ++b)
            if (b < nc) v[b] = (node[b] ? lab_n_in : lab_e_in)[out[b] * n_lab + q];
#pragma unroll
          for (int b = 0; b < CB; ++b)
            if (b < nc) buf[b * n_lab + q] = v[b];
        }
        wave_lds_order();
        // entries from their CG terms, written where the template has an orbital
        for (int t = lane; t < n_lab; t += kLW) {
          const int r = t / nf, c = t - r * nf;
          float acc[CB];
#pragma unroll
          for (int b = 0; b < CB; ++b) acc[b] = 0.0f;
          const int t1 = t_start[t + 1];
          for (int k = t_start[t]; k < t1; ++k) {
            const float cf = t_coef[k];
            const int ix = t_idx[k];
#pragma unroll
            for (int b = 0; b < CB; ++b) acc[b] += cf * buf[b * n_lab + ix];
          }
#pragma unroll
          for (int b = 0; b < CB; ++b) {
            const int lr = omap[zi[b] * nf + r], lc = omap[zj[b] * nf + c];
            if (b < nc && ok[b] && lr >= 0 && lc >= 0) Hout[base[b] + static_cast<int64_t>(lr) * ld[b] + lc] = acc[b];
          }
        }
        wave_lds_order();
      }
    }
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
  const int n_terms = to_label ? info.lab_terms : info.ent_terms;
  const int64_t rows = (edges ? g->n_edges : 0) + (nodes ? o->n_atoms : 0);
  // algorithmic bytes: every label row once, and every matrix entry once
  // when the graph covers each block (a fully connected structure)
  Timed tm(stream, to_label ? "matrix_to_label" : "label_to_matrix", 0.0,
           4.0 * (double(rows) * info.n_lab + double(h_elems)));
  int64_t blocks = (static_cast<int64_t>(o->n_atoms) + kLWaves - 1) / kLWaves;
  if (blocks > 2048) blocks = 2048;
  const size_t base_words = lds_words(info.n_lab, n_terms, info.n_species, info.n_full);
  auto launch = [&](auto cb) -> egnn_status {
    constexpr int CB = decltype(cb)::value;
    const size_t smem = 4 * (base_words + static_cast<size_t>(kLWaves) * CB * info.n_lab);
    if (smem > 160 * 1024) {
      set_error("Matrix <-> Label needs %zu bytes of LDS; reduce the basis", smem);
      return EGNN_E_UNSUPPORTED;
    }
    if (to_label)
      labels_kernel<CB, true><<<static_cast<unsigned>(blocks), kLW * kLWaves, smem, stream>>>(
          slot, R, Hin, nullptr, nullptr, nullptr, le_out, ln_out, skip);
    else
      labels_kernel<CB, false><<<static_cast<unsigned>(blocks), kLW * kLWaves, smem, stream>>>(
          slot, R, nullptr, Hout, le_in, ln_in, nullptr, nullptr, skip);
    EGNN_CHECK_LAUNCH();
    return EGNN_OK;
  };
  if (info.n_lab <= 512) return launch(std::integral_constant<int, 8>{});
  return launch(std::integral_constant<int, 4>{});
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
