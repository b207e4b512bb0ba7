// Status text, thread-local error detail and layer shape bookkeeping.
#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace egnn {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

bool make_shape(const egnn_layer_desc *d, LayerShape *s) {
  if (!d) return false;
  if (d->lmax < 1 || d->lmax > 8 || (d->lmax > 4 && d->lmax != 6 && d->lmax != 8)) return false;  // 1..4, 6, 8
  if (d->mmax < 0 || d->mmax > d->lmax || d->mmax > 2) return false;
  if (d->C < 8 || d->C > 256 || d->C % 8 != 0) return false;
  if (d->n_rbf < 2 || d->n_rbf > 16) return false;
  if (!(d->r_cut > 0.0)) return false;
  if (d->storage != EGNN_F32 && d->storage != EGNN_BF16) return false;
  s->lmax = d->lmax;
  s->mmax = d->mmax;
  s->C = d->C;
  s->n_rbf = d->n_rbf;
  s->K = (d->lmax + 1) * (d->lmax + 1);
  s->n_pairs = pair_count(d->lmax, d->mmax);
  s->nD = d_count(d->lmax, d->mmax);
  int raw = s->nD + s->n_rbf + 1;  // + destination row
  s->gstride = (raw + 15) / 16 * 16;
  s->kept = kept_count(d->lmax, d->mmax);
  for (int m = 0; m < 3; ++m) {
    if (m > d->mmax) {
      s->Kg[m] = s->Ng[m] = 0;
      continue;
    }
    int nl = d->lmax - m + 1;
    int sides = m == 0 ? 1 : 2;
    s->Kg[m] = sides * nl * 2 * d->C;
    s->Ng[m] = sides * nl * d->C;
  }
  s->r_cut = static_cast<float>(d->r_cut);
  s->storage = d->storage;
  return true;
}

}  // namespace egnn

using namespace egnn;

extern "C" const char *egnn_status_string(int status) {
  switch (status) {
    case EGNN_OK: return "ok";
    case EGNN_E_ARG: return "invalid argument";
    case EGNN_E_CAPACITY: return "graph capacity too small";
    case EGNN_E_HIP: return "HIP runtime error";
    case EGNN_E_UNSUPPORTED: return "unsupported request";
    case EGNN_E_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

extern "C" const char *egnn_last_error(void) { return g_err; }

extern "C" int egnn_version(void) { return 100; }

extern "C" size_t egnn_layer_weight_count(const egnn_layer_desc *d) {
  LayerShape s;
  if (!make_shape(d, &s)) return 0;
  size_t n = 0;
  for (int m = 0; m <= s.mmax; ++m) {
    size_t nl = s.lmax - m + 1;
    size_t blk = (nl * s.C) * (nl * 2 * s.C);
    n += m == 0 ? blk : 2 * blk;
  }
  n += static_cast<size_t>(s.n_rbf) * s.n_pairs * 2 * s.C;
  n += s.C;
  return n;
}

extern "C" int32_t egnn_geom_stride(const egnn_layer_desc *d) {
  LayerShape s;
  if (!make_shape(d, &s)) return 0;
  return s.gstride;
}
