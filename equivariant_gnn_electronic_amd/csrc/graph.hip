// Periodic / open cell-list neighbour builder emitting a destination-sorted CSR.
//
// The graph is the cutoff graph of the structure stored by destination: every
// atom owns the edges directed into it (review of arXiv 2507.03840, "What
// carries the argument"; MALOQ Sec. III-D "target-nodes-own-edges").  Periodic
// axes follow the DFT cell (MALOQ Sec. III-D2).
//
// Design: atoms are binned into cells no smaller than the cutoff; each row is
// enumerated by one 64-lane wave over the stencil of neighbouring cells, in
// two passes (count, then fill) so no edge list is ever over-allocated.  The
// distance test is fp64 with contraction disabled, so the edge set is exactly
// the one the stated predicate defines.  Rows are then rank-sorted by
// (source, image) and the source grouping is rank-sorted by edge id, which
// makes every output array deterministic although the cell lists and the
// fill order use integer atomics.
#pragma clang fp contract(off)

#include <climits>
#include <mutex>

#include "common.h"
#include "timing.h"

namespace egnn {
namespace {

constexpr int kWave = 64;
constexpr int kScanThreads = 1024;

struct Grid {
  double lo[3], box[3], h[3];
  int n[3];
  int reach[3];
  int periodic[3];
  int n_cells;
};

bool make_grid(const double lo[3], const double box[3], uint32_t mask, double r_cut, Grid *g) {
  int64_t total = 1;
  for (int a = 0; a < 3; ++a) {
    if (!(box[a] > 0.0) || !(r_cut > 0.0)) return false;
    g->lo[a] = lo[a];
    g->box[a] = box[a];
    g->periodic[a] = (mask >> a) & 1u;
    // cells a hair wider than the cutoff, so that fp64 rounding of the cell
    // index can never hide a pair that is within the cutoff
    double wide = r_cut * (1.0 + 1e-9);
    int64_t n = static_cast<int64_t>(box[a] / wide);
    if (n < 1) n = 1;
    if (n > 512) n = 512;
    g->n[a] = static_cast<int>(n);
    g->h[a] = box[a] / static_cast<double>(n);
    int reach = static_cast<int>(ceil(wide / g->h[a]));
    if (reach < 1) reach = 1;
    g->reach[a] = reach;
    total *= n;
  }
  g->n_cells = static_cast<int>(total);
  return true;
}

struct Ws {
  int *cell_count, *cell_start, *cell_cursor, *cell_atoms;
  int *ucell;          // [n_src][3] unwrapped cell index of each stored position
  int *atom_cell;      // [n_src]
  int *row_count;      // [n_dst]
  int *src_count, *src_cursor;  // [n_src]
  int *scalars;        // [0] E, [1] max row, [2] error flags, [3] max src group
  unsigned long long *keys;     // [capacity]
  size_t bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Ws carve(void *base, int n_dst, int n_src, int n_cells, int64_t capacity) {
  Ws w{};
  char *p = static_cast<char *>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) { char *r = p ? p + o : nullptr; o += align256(bytes); return r; };
  w.cell_count = reinterpret_cast<int *>(take(sizeof(int) * n_cells));
  w.cell_start = reinterpret_cast<int *>(take(sizeof(int) * (n_cells + 1)));
  w.cell_cursor = reinterpret_cast<int *>(take(sizeof(int) * n_cells));
  w.cell_atoms = reinterpret_cast<int *>(take(sizeof(int) * n_src));
  w.ucell = reinterpret_cast<int *>(take(sizeof(int) * 3 * n_src));
  w.atom_cell = reinterpret_cast<int *>(take(sizeof(int) * n_src));
  w.row_count = reinterpret_cast<int *>(take(sizeof(int) * (n_dst + 1)));
  w.src_count = reinterpret_cast<int *>(take(sizeof(int) * (n_src + 1)));
  w.src_cursor = reinterpret_cast<int *>(take(sizeof(int) * (n_src + 1)));
  w.scalars = reinterpret_cast<int *>(take(sizeof(int) * 16));
  w.keys = reinterpret_cast<unsigned long long *>(take(sizeof(unsigned long long) * (capacity > 0 ? capacity : 1)));
  w.bytes = o;
  return w;
}

__global__ void fill_int(int *p, int n, int v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Exclusive scan of in[0..n) into out[0..n] (out[n] = total) by one
// workgroup; also records max(in) into *maxv.
__global__ void __launch_bounds__(kScanThreads) scan_exclusive(const int *in, int *out, int n,
                                                               int *total, int *maxv) {
  __shared__ int part[kScanThreads];
  int carry = 0, mx = 0;
  for (int base = 0; base < n; base += kScanThreads * 4) {
    int v[4];
    int s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int i = base + threadIdx.x * 4 + j;
      v[j] = i < n ? in[i] : 0;
      s += v[j];
      mx = max(mx, v[j]);
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
      int t = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += t;
      __syncthreads();
    }
    int run = carry + part[threadIdx.x] - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int i = base + threadIdx.x * 4 + j;
      if (i < n) out[i] = run;
      run += v[j];
    }
    carry += part[kScanThreads - 1];
    __syncthreads();
  }
  // max over the workgroup
  part[threadIdx.x] = mx;
  __syncthreads();
  for (int off = kScanThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] = max(part[threadIdx.x], part[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[n] = carry;
    if (total) *total = carry;
    if (maxv) *maxv = part[0];
  }
}

__device__ inline int cell_flat(const Grid &g, int wx, int wy, int wz) {
  return (wx * g.n[1] + wy) * g.n[2] + wz;
}

__global__ void bin_atoms(const double *pos, int n_src, Grid g, int *ucell, int *atom_cell,
                          int *cell_count, int *flags) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_src) return;
  int w[3];
  for (int a = 0; a < 3; ++a) {
    double t = floor((pos[3 * s + a] - g.lo[a]) / g.h[a]);
    if (!(t > -1e8 && t < 1e8)) {  // non-finite or absurdly far position
      atomicOr(flags, 1);
      t = 0.0;
    }
    int u = static_cast<int>(t);
    if (g.periodic[a]) {
      int m = u % g.n[a];
      w[a] = m < 0 ? m + g.n[a] : m;
    } else {
      u = u < 0 ? 0 : (u >= g.n[a] ? g.n[a] - 1 : u);
      w[a] = u;
    }
    ucell[3 * s + a] = u;
  }
  int c = cell_flat(g, w[0], w[1], w[2]);
  atom_cell[s] = c;
  atomicAdd(&cell_count[c], 1);
}

__global__ void scatter_atoms(int n_src, const int *atom_cell, const int *cell_start, int *cell_cursor,
                              int *cell_atoms) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_src) return;
  int c = atom_cell[s];
  int slot = atomicAdd(&cell_cursor[c], 1);
  cell_atoms[cell_start[c] + slot] = s;
}

// The exact predicate: p = x_s + S*L; delta = x_d - p; d2 = (dx^2 + dy^2) + dz^2.
struct PairTest {
  double dx, dy, dz, d2;
};
__device__ inline PairTest pair_test(const double *pos, int d, int s, int Sx, int Sy, int Sz, const Grid &g) {
  PairTest t;
  double px = pos[3 * s + 0] + static_cast<double>(Sx) * g.box[0];
  double py = pos[3 * s + 1] + static_cast<double>(Sy) * g.box[1];
  double pz = pos[3 * s + 2] + static_cast<double>(Sz) * g.box[2];
  t.dx = pos[3 * d + 0] - px;
  t.dy = pos[3 * d + 1] - py;
  t.dz = pos[3 * d + 2] - pz;
  double a = t.dx * t.dx;
  double b = t.dy * t.dy;
  double c = t.dz * t.dz;
  t.d2 = (a + b) + c;
  return t;
}

__device__ inline unsigned long long make_key(int s, int Sx, int Sy, int Sz) {
  return (static_cast<unsigned long long>(static_cast<unsigned>(s)) << 24) |
         (static_cast<unsigned long long>(Sx + 128) << 16) |
         (static_cast<unsigned long long>(Sy + 128) << 8) | static_cast<unsigned long long>(Sz + 128);
}

// Enumerate the candidates of row d (one wave); MODE 0 counts, MODE 1 appends keys.
template <int MODE>
__global__ void __launch_bounds__(256) row_pass(const double *pos, int n_dst, Grid g, double rc2,
                                                const int *ucell, const int *cell_start,
                                                const int *cell_atoms, int *row_count,
                                                const int *row_ptr, unsigned long long *keys,
                                                int *flags) {
  const int lane = threadIdx.x & (kWave - 1);
  const int d = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (d >= n_dst) return;
  const int ud[3] = {ucell[3 * d], ucell[3 * d + 1], ucell[3 * d + 2]};
  int count = 0;
  const int base = MODE == 1 ? row_ptr[d] : 0;
  for (int ox = -g.reach[0]; ox <= g.reach[0]; ++ox) {
    int ux = ud[0] + ox;
    if (!g.periodic[0] && (ux < 0 || ux >= g.n[0])) continue;
    int wx = g.periodic[0] ? ((ux % g.n[0]) + g.n[0]) % g.n[0] : ux;
    for (int oy = -g.reach[1]; oy <= g.reach[1]; ++oy) {
      int uy = ud[1] + oy;
      if (!g.periodic[1] && (uy < 0 || uy >= g.n[1])) continue;
      int wy = g.periodic[1] ? ((uy % g.n[1]) + g.n[1]) % g.n[1] : uy;
      for (int oz = -g.reach[2]; oz <= g.reach[2]; ++oz) {
        int uz = ud[2] + oz;
        if (!g.periodic[2] && (uz < 0 || uz >= g.n[2])) continue;
        int wz = g.periodic[2] ? ((uz % g.n[2]) + g.n[2]) % g.n[2] : uz;
        int c = cell_flat(g, wx, wy, wz);
        int b = cell_start[c], e = cell_start[c + 1];
        for (int i = b; i < e; i += kWave) {
          int j = i + lane;
          bool pass = false;
          int s = 0, Sx = 0, Sy = 0, Sz = 0;
          if (j < e) {
            s = cell_atoms[j];
            if (g.periodic[0]) Sx = (ux - ucell[3 * s + 0]) / g.n[0];
            if (g.periodic[1]) Sy = (uy - ucell[3 * s + 1]) / g.n[1];
            if (g.periodic[2]) Sz = (uz - ucell[3 * s + 2]) / g.n[2];
            PairTest t = pair_test(pos, d, s, Sx, Sy, Sz, g);
            pass = (t.d2 < rc2) && !(s == d && Sx == 0 && Sy == 0 && Sz == 0);
            if (pass && (Sx < -127 || Sx > 127 || Sy < -127 || Sy > 127 || Sz < -127 || Sz > 127)) {
              atomicOr(flags, 2);
              pass = false;
            }
          }
          unsigned long long m = __ballot(pass);
          if (MODE == 1 && pass) {
            int before = __popcll(m & ((1ull << lane) - 1ull));
            keys[base + count + before] = make_key(s, Sx, Sy, Sz);
          }
          count += __popcll(m);
        }
      }
    }
  }
  if (MODE == 0 && lane == 0) row_count[d] = count;
}

// Rank-sort each row by key and write the edge arrays (one wave per row).
__global__ void __launch_bounds__(256) row_sort_write(const double *pos, int n_dst, Grid g,
                                                      const int *row_ptr,
                                                      const unsigned long long *keys, int *src,
                                                      int8_t *shift, float *vec, float *dist) {
  const int lane = threadIdx.x & (kWave - 1);
  const int d = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (d >= n_dst) return;
  const int b = row_ptr[d], n = row_ptr[d + 1] - b;
  for (int i = lane; i < n; i += kWave) {
    unsigned long long ki = keys[b + i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += keys[b + j] < ki ? 1 : 0;
    int s = static_cast<int>(ki >> 24);
    int Sx = static_cast<int>((ki >> 16) & 0xFF) - 128;
    int Sy = static_cast<int>((ki >> 8) & 0xFF) - 128;
    int Sz = static_cast<int>(ki & 0xFF) - 128;
    PairTest t = pair_test(pos, d, s, Sx, Sy, Sz, g);
    int o = b + rank;
    src[o] = s;
    shift[3 * o + 0] = static_cast<int8_t>(Sx);
    shift[3 * o + 1] = static_cast<int8_t>(Sy);
    shift[3 * o + 2] = static_cast<int8_t>(Sz);
    vec[3 * o + 0] = static_cast<float>(t.dx);
    vec[3 * o + 1] = static_cast<float>(t.dy);
    vec[3 * o + 2] = static_cast<float>(t.dz);
    dist[o] = static_cast<float>(sqrt(t.d2));
  }
}

__global__ void src_count_kernel(const int *src, int64_t E, int *src_count) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < E) atomicAdd(&src_count[src[e]], 1);
}

__global__ void src_fill_kernel(const int *src, int64_t E, const int *src_ptr, int *src_cursor, int *tmp) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int s = src[e];
  int slot = atomicAdd(&src_cursor[s], 1);
  tmp[src_ptr[s] + slot] = static_cast<int>(e);
}

__global__ void __launch_bounds__(256) src_sort_kernel(int n_src, const int *src_ptr, const int *tmp,
                                                       int *src_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (s >= n_src) return;
  const int b = src_ptr[s], n = src_ptr[s + 1] - b;
  for (int i = lane; i < n; i += kWave) {
    int ei = tmp[b + i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += tmp[b + j] < ei ? 1 : 0;
    src_perm[b + rank] = ei;
  }
}

constexpr int kMaxGroup = 65535;

// Source grouping of a caller's CSR: sources outside [0, n_src) are left out.
__global__ void src_count_checked(const int *src, int64_t E, int n_src, int *src_count) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int s = src[e];
  if (s >= 0 && s < n_src) atomicAdd(&src_count[s], 1);
}

__global__ void src_fill_checked(const int *src, int64_t E, int n_src, const int *src_ptr, int *src_cursor,
                                 int *tmp) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int s = src[e];
  if (s < 0 || s >= n_src) return;
  const int slot = atomicAdd(&src_cursor[s], 1);
  tmp[src_ptr[s] + slot] = static_cast<int>(e);
}

struct GroupWs {
  int *src_count, *src_cursor, *tmp;
  size_t bytes;
};

GroupWs carve_group(void *base, int n_src, int64_t E) {
  GroupWs w{};
  char *p = static_cast<char *>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) { char *r = p ? p + o : nullptr; o += align256(bytes); return r; };
  w.src_count = reinterpret_cast<int *>(take(sizeof(int) * (n_src + 1)));
  w.src_cursor = reinterpret_cast<int *>(take(sizeof(int) * (n_src + 1)));
  w.tmp = reinterpret_cast<int *>(take(sizeof(int) * (E > 0 ? E : 1)));
  w.bytes = o;
  return w;
}

}  // namespace
}  // namespace egnn

using namespace egnn;

extern "C" egnn_status egnn_build_graph_workspace(int32_t n_dst, int32_t n_src, const double lo[3],
                                                  const double box[3], uint32_t periodic_mask,
                                                  double r_cut, int64_t capacity, size_t *bytes) {
  clear_error();
  EGNN_REQUIRE(lo && box && bytes, "null argument");
  EGNN_REQUIRE(n_dst >= 0 && n_src >= n_dst, "need 0 <= n_dst <= n_src (got %d, %d)", n_dst, n_src);
  EGNN_REQUIRE(capacity >= 0, "negative capacity");
  EGNN_REQUIRE(periodic_mask < 8, "periodic_mask has bits above axis 2");
  Grid g;
  EGNN_REQUIRE(make_grid(lo, box, periodic_mask, r_cut, &g), "box and r_cut must be positive");
  *bytes = carve(nullptr, n_dst, n_src, g.n_cells, capacity).bytes;
  return EGNN_OK;
}

namespace egnn {
namespace {

// Scratch of the allocation-free variant: one copy per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (in host
// code the name is a host-side stand-in); it asks the runtime for the
// device's address once per device and uses that address only.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// Address of the current device's scratch (looked up on its first use there).
egnn_status noalloc_scratch(void **out) {
  int dev = -1;
  EGNN_TRY_HIP(hipGetDevice(&dev));
  EGNN_REQUIRE(dev >= 0 && dev < kMaxDevices, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    EGNN_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    EGNN_REQUIRE(p != nullptr, "no device address for the scratch array");
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return EGNN_OK;
}

egnn_status build_graph_impl(const double *pos, const double lo[3], const double box[3], uint32_t periodic_mask,
                             double r_cut, egnn_graph *gr, void *ws, size_t ws_bytes, hipStream_t stream);

}  // namespace
}  // namespace egnn

extern "C" egnn_status egnn_build_graph(const double *pos, const double lo[3], const double box[3],
                                        uint32_t periodic_mask, double r_cut, egnn_graph *gr, void *ws,
                                        size_t ws_bytes, hipStream_t stream) {
  clear_error();
  return build_graph_impl(pos, lo, box, periodic_mask, r_cut, gr, ws, ws_bytes, stream);
}

extern "C" egnn_status egnn_build_graph_noalloc(const double *pos, const double lo[3], const double box[3],
                                                uint32_t periodic_mask, double r_cut, egnn_graph *gr,
                                                hipStream_t stream) {
  clear_error();
  EGNN_REQUIRE(gr && lo && box, "null argument");
  EGNN_REQUIRE(gr->n_dst >= 0 && gr->n_src >= gr->n_dst, "need 0 <= n_dst <= n_src (got %d, %d)", gr->n_dst,
               gr->n_src);
  EGNN_REQUIRE(gr->capacity >= 0, "negative capacity");
  Grid g;
  EGNN_REQUIRE(make_grid(lo, box, periodic_mask, r_cut, &g), "box and r_cut must be positive");
  const size_t need = carve(nullptr, gr->n_dst, gr->n_src, g.n_cells, gr->capacity).bytes;
  if (need > kNoAllocScratchBytes) {
    set_error("needs %zu bytes of workspace; the allocation-free variant has %zu (fewer edges of capacity, "
              "fewer atoms or cells, or egnn_build_graph with a workspace)", need, kNoAllocScratchBytes);
    return EGNN_E_WORKSPACE;
  }
  void *ws = nullptr;
  egnn_status st = noalloc_scratch(&ws);
  if (st != EGNN_OK) return st;
  return build_graph_impl(pos, lo, box, periodic_mask, r_cut, gr, ws, kNoAllocScratchBytes, stream);
}

namespace egnn {
namespace {

egnn_status build_graph_impl(const double *pos, const double lo[3], const double box[3], uint32_t periodic_mask,
                             double r_cut, egnn_graph *gr, void *ws, size_t ws_bytes, hipStream_t stream) {
  EGNN_REQUIRE(gr && lo && box, "null argument");
  const int n_dst = gr->n_dst, n_src = gr->n_src;
  EGNN_REQUIRE(n_dst >= 0 && n_src >= n_dst, "need 0 <= n_dst <= n_src (got %d, %d)", n_dst, n_src);
  EGNN_REQUIRE(gr->capacity >= 0, "negative capacity");
  EGNN_REQUIRE(periodic_mask < 8, "periodic_mask has bits above axis 2");
  EGNN_REQUIRE(gr->row_ptr && gr->src_ptr, "row_ptr or src_ptr is null");
  EGNN_REQUIRE(n_src == 0 || pos, "pos is null");
  Grid g;
  EGNN_REQUIRE(make_grid(lo, box, periodic_mask, r_cut, &g), "box and r_cut must be positive");
  const int64_t cap = gr->capacity;
  Ws w = carve(ws, n_dst, n_src, g.n_cells, cap);
  if (!ws || ws_bytes < w.bytes) {
    set_error("workspace of %zu bytes, need %zu", ws_bytes, w.bytes);
    return EGNN_E_WORKSPACE;
  }
  if (cap > 0) {
    EGNN_REQUIRE(gr->src && gr->shift && gr->vec && gr->dist && gr->src_perm,
                 "edge arrays must be non-null when capacity > 0");
  }
  const double rc2 = r_cut * r_cut;
  const int T = 256;
  const int rows_per_block = T / kWave;
  {
  Timed t_count(stream, "graph_count", 0.0, double(n_src) * 24.0 + double(n_dst) * 4.0);
  // cells
  fill_int<<<ceil_div(g.n_cells, T), T, 0, stream>>>(w.cell_count, g.n_cells, 0);
  fill_int<<<ceil_div(g.n_cells, T), T, 0, stream>>>(w.cell_cursor, g.n_cells, 0);
  fill_int<<<1, 16, 0, stream>>>(w.scalars, 16, 0);
  if (n_src > 0)
    bin_atoms<<<ceil_div(n_src, T), T, 0, stream>>>(pos, n_src, g, w.ucell, w.atom_cell, w.cell_count,
                                                    w.scalars + 2);
  scan_exclusive<<<1, kScanThreads, 0, stream>>>(w.cell_count, w.cell_start, g.n_cells, nullptr, nullptr);
  if (n_src > 0)
    scatter_atoms<<<ceil_div(n_src, T), T, 0, stream>>>(n_src, w.atom_cell, w.cell_start, w.cell_cursor,
                                                        w.cell_atoms);
  // rows: count, scan
  if (n_dst > 0)
    row_pass<0><<<ceil_div(n_dst, rows_per_block), T, 0, stream>>>(
        pos, n_dst, g, rc2, w.ucell, w.cell_start, w.cell_atoms, w.row_count, nullptr, nullptr, w.scalars + 2);
  scan_exclusive<<<1, kScanThreads, 0, stream>>>(w.row_count, gr->row_ptr, n_dst, w.scalars + 0, w.scalars + 1);
  EGNN_CHECK_LAUNCH();
  }
  int host[4];
  EGNN_TRY_HIP(hipMemcpyAsync(host, w.scalars, sizeof(host), hipMemcpyDeviceToHost, stream));
  EGNN_TRY_HIP(hipStreamSynchronize(stream));
  const int64_t E = host[0];
  gr->n_edges = E;
  if (host[2] & 1) {
    set_error("a position is not finite or lies absurdly far from the cell");
    return EGNN_E_ARG;
  }
  if (host[2] & 2) {
    set_error("an image shift exceeds the int8 range (cutoff far larger than the cell)");
    return EGNN_E_UNSUPPORTED;
  }
  if (host[1] > kMaxGroup) {
    set_error("a row has %d edges; at most %d are supported", host[1], kMaxGroup);
    return EGNN_E_UNSUPPORTED;
  }
  if (E > cap) {
    set_error("graph needs %lld edges, capacity is %lld", static_cast<long long>(E),
              static_cast<long long>(cap));
    return EGNN_E_CAPACITY;
  }
  // rows: fill keys, sort, write
  Timed t_fill(stream, "graph_fill", 0.0, double(E) * (4.0 + 3.0 + 12.0 + 4.0 + 4.0) + double(n_src) * 4.0);
  if (n_dst > 0 && E > 0) {
    row_pass<1><<<ceil_div(n_dst, rows_per_block), T, 0, stream>>>(
        pos, n_dst, g, rc2, w.ucell, w.cell_start, w.cell_atoms, nullptr, gr->row_ptr, w.keys, w.scalars + 2);
    row_sort_write<<<ceil_div(n_dst, rows_per_block), T, 0, stream>>>(pos, n_dst, g, gr->row_ptr, w.keys,
                                                                     gr->src, gr->shift, gr->vec, gr->dist);
  }
  // source grouping
  fill_int<<<ceil_div(n_src + 1, T), T, 0, stream>>>(w.src_count, n_src + 1, 0);
  fill_int<<<ceil_div(n_src + 1, T), T, 0, stream>>>(w.src_cursor, n_src + 1, 0);
  if (E > 0) src_count_kernel<<<ceil_div(E, T), T, 0, stream>>>(gr->src, E, w.src_count);
  scan_exclusive<<<1, kScanThreads, 0, stream>>>(w.src_count, gr->src_ptr, n_src, nullptr, w.scalars + 3);
  if (E > 0) {
    int *tmp = reinterpret_cast<int *>(w.keys);
    src_fill_kernel<<<ceil_div(E, T), T, 0, stream>>>(gr->src, E, gr->src_ptr, w.src_cursor, tmp);
    src_sort_kernel<<<ceil_div(n_src, rows_per_block), T, 0, stream>>>(n_src, gr->src_ptr, tmp, gr->src_perm);
  }
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}

}  // namespace
}  // namespace egnn

extern "C" egnn_status egnn_group_sources_workspace(int32_t n_src, int64_t n_edges, size_t *bytes) {
  clear_error();
  EGNN_REQUIRE(bytes, "null argument");
  EGNN_REQUIRE(n_src >= 0, "negative source count");
  EGNN_REQUIRE(n_edges >= 0 && n_edges <= INT_MAX, "n_edges must be 0..2^31 - 1");
  *bytes = carve_group(nullptr, n_src, n_edges).bytes;
  return EGNN_OK;
}

extern "C" egnn_status egnn_group_sources(egnn_graph *gr, void *ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  EGNN_REQUIRE(gr, "graph is null");
  EGNN_REQUIRE(gr->n_src >= 0, "negative source count");
  EGNN_REQUIRE(gr->n_edges >= 0 && gr->n_edges <= INT_MAX, "n_edges must be 0..2^31 - 1");
  EGNN_REQUIRE(gr->src_ptr, "src_ptr is null");
  const int n_src = gr->n_src;
  const int64_t E = gr->n_edges;
  if (E > 0) EGNN_REQUIRE(gr->src && gr->src_perm, "src or src_perm is null");
  GroupWs w = carve_group(ws, n_src, E);
  if (!ws || ws_bytes < w.bytes) {
    set_error("workspace of %zu bytes, need %zu", ws_bytes, w.bytes);
    return EGNN_E_WORKSPACE;
  }
  constexpr int T = 256;
  const int rows_per_block = T / kWave;
  Timed t(stream, "group_sources", 0.0, double(E) * 4.0 * 3.0 + double(n_src) * 4.0);
  fill_int<<<ceil_div(n_src + 1, T), T, 0, stream>>>(w.src_count, n_src + 1, 0);
  fill_int<<<ceil_div(n_src + 1, T), T, 0, stream>>>(w.src_cursor, n_src + 1, 0);
  if (E > 0) src_count_checked<<<ceil_div(E, T), T, 0, stream>>>(gr->src, E, n_src, w.src_count);
  scan_exclusive<<<1, kScanThreads, 0, stream>>>(w.src_count, gr->src_ptr, n_src, nullptr, nullptr);
  if (E > 0 && n_src > 0) {
    src_fill_checked<<<ceil_div(E, T), T, 0, stream>>>(gr->src, E, n_src, gr->src_ptr, w.src_cursor, w.tmp);
    src_sort_kernel<<<ceil_div(n_src, rows_per_block), T, 0, stream>>>(n_src, gr->src_ptr, w.tmp, gr->src_perm);
  }
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}
