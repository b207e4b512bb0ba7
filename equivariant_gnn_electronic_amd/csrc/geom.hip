// "Compute Wigners": per-edge Wigner rows and radial basis (MALOQ Sec. III-C,
// Fig. 3(c): Euler angles of the edge, then the (2l+1)^2 entries of D^l).
//
// The pages fuse this chain into one Triton kernel built on tensor-core
// matrix products.  Here each thread owns one edge and runs the
// Ivanic-Ruedenberg recursion in registers (about a thousand fp32 FMAs per
// edge at lmax 4), so the kernel is bound by writing the result: only the
// rows |m| <= mmax that the layer consumes are stored, plus the radial basis.
#include "common.h"
#include "wigner.h"
#include "timing.h"

namespace egnn {
namespace {

// Destination row of every edge: one wave per row, its lanes over the row's edges.
__global__ void edge_dst_kernel(const int *row_ptr, int n_dst, int stride, int col, float *geom) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int d = static_cast<int>(t / 64), lane = static_cast<int>(t % 64);
  if (d >= n_dst) return;
  const int e1 = row_ptr[d + 1];
  for (int e = row_ptr[d] + lane; e < e1; e += 64)
    reinterpret_cast<int *>(geom)[static_cast<int64_t>(e) * stride + col] = d;
}

template <int LMAX, int MMAX>
__global__ void __launch_bounds__(256) edge_geom_kernel(const float *vec, const float *dist, int64_t E,
                                                        int n_rbf, float r_cut, int stride, float *geom) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float R[3][3];
  edge_rotation(vec[3 * e], vec[3 * e + 1], vec[3 * e + 2], R);
  constexpr int ND = d_count(LMAX, MMAX);
  float D[ND];
  wigner_rows<LMAX, MMAX>(R, D);
  const float r = dist[e];
  float rb[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) rb[k] = k < n_rbf ? rbf_value(r, k, n_rbf, r_cut) : 0.0f;
  // The row leaves as 16-byte stores (the stride is a multiple of 16 floats),
  // a quarter of the store instructions of one float at a time: 0.135 ->
  // 0.102 ms on the HfO2 graph.  The destination column is written
  // afterwards by edge_dst_kernel.
  constexpr int SMAX = (ND + 16 + 1 + 15) / 16 * 16;
  float4 *o4 = reinterpret_cast<float4 *>(geom + e * stride);
#pragma unroll
  for (int q = 0; q < SMAX / 4; ++q) {
    if (4 * q >= stride) break;
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = 4 * q + t;
      float x = 0.0f;
      if (j < ND) x = D[j];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (j == ND + k) x = rb[k];
      v[t] = x;
    }
    o4[q] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int LMAX, int MMAX>
void launch_geom(const egnn_graph *g, const LayerShape &s, float *geom, hipStream_t st) {
  const int T = 256;
  edge_geom_kernel<LMAX, MMAX><<<ceil_div(g->n_edges, T), T, 0, st>>>(g->vec, g->dist, g->n_edges, s.n_rbf,
                                                                     s.r_cut, s.gstride, geom);
  edge_dst_kernel<<<ceil_div(static_cast<int64_t>(g->n_dst) * 64, T), T, 0, st>>>(g->row_ptr, g->n_dst, s.gstride,
                                                                                 s.nD + s.n_rbf, geom);
}

}  // namespace

}  // namespace egnn

using namespace egnn;

extern "C" egnn_status egnn_edge_geom(const egnn_layer_desc *d, const egnn_graph *g, float *geom,
                                      hipStream_t stream) {
  clear_error();
  LayerShape s;
  EGNN_REQUIRE(make_shape(d, &s), "invalid layer description");
  EGNN_REQUIRE(g, "graph is null");
  EGNN_REQUIRE(g->n_edges >= 0 && g->n_edges <= g->capacity, "graph n_edges out of range");
  if (g->n_edges == 0) return EGNN_OK;
  EGNN_REQUIRE(geom && g->vec && g->dist && g->row_ptr, "null pointer");
  EGNN_REQUIRE(reinterpret_cast<uintptr_t>(geom) % 16 == 0, "geom must be 16-byte aligned (rows are written as 16-byte stores)");
  Timed t(stream, "edge_geom", 0.0, double(g->n_edges) * (16.0 + s.gstride * 4.0));
  EGNN_DISPATCH_LM(s.lmax, s.mmax, launch_geom, g, s, geom, stream);
  EGNN_CHECK_LAUNCH();
  return EGNN_OK;
}
