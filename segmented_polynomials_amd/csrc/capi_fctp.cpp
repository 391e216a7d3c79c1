// C ABI of the fully connected (uvw) tensor product: descriptor, the three
// GEMM passes' tables, the weight-gradient tables, validation, launches.
// Host code.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "capi_util.hpp"
#include "cg.hpp"
#include "fcconv_tables.hpp"
#include "fctp_ps_tables.hpp"
#include "fctp_tables.hpp"
#include "irreps.hpp"
#include "launch.hpp"
#include "linear_tables.hpp"
#include "segpoly.h"

using namespace segpoly;

namespace {

constexpr size_t kLdsLimit = 52 * 1024;  // per workgroup (three workgroups fit a CU's 160 KB)
// The float 32-column product kernels run four workgroups per CU.
size_t product_lds_limit(int dtype, int tn) { return dtype == SEGPOLY_F32 && tn == 32 ? 40 * 1024 : kLdsLimit; }
constexpr int kMaxL = 6;

// A term without a parity letter is an SO(3) irrep (parity 0: the parity
// rule p3 = p1 p2 then holds for every triple); mixing the two is an error.
std::vector<Irrep> parse_any(const std::string& s) {
  try {
    return parse_irreps(s);
  } catch (const ParseError&) {
  }
  std::vector<Irrep> out;
  size_t start = 0;
  while (true) {
    const size_t plus = s.find('+', start);
    std::string term = s.substr(start, plus == std::string::npos ? std::string::npos : plus - start);
    term.erase(std::remove_if(term.begin(), term.end(), [](unsigned char c) { return std::isspace(c); }), term.end());
    int mul = 1;
    const size_t x = term.find('x');
    std::string ls = term;
    if (x != std::string::npos) {
      const std::string m = term.substr(0, x);
      if (m.empty() || m.size() > 6 || !std::all_of(m.begin(), m.end(), ::isdigit))
        throw ParseError("bad multiplicity in irreps term '" + term + "'");
      mul = std::stoi(m);
      ls = term.substr(x + 1);
    }
    if (ls.empty() || ls.size() > 3 || !std::all_of(ls.begin(), ls.end(), ::isdigit))
      throw ParseError("bad irreps term '" + term + "' (expected MULxLP with P in {e, o}, or MULxL for SO(3))");
    out.push_back({mul, std::stoi(ls), 0});
    if (plus == std::string::npos) break;
    start = plus + 1;
  }
  return out;
}

std::vector<int64_t> offsets(const std::vector<Irrep>& v) {
  std::vector<int64_t> o(v.size() + 1, 0);
  for (size_t i = 0; i < v.size(); ++i) o[i + 1] = o[i] + static_cast<int64_t>(v[i].mul) * (2 * v[i].l + 1);
  return o;
}

struct FcPass {
  std::vector<FcRes> res;
  std::vector<FcTerm> terms;
  int tn = 32;
  int nt = 1;                        // entry class of the launch
  bool lds_direct = false;           // every term suits LDS-direct weight chunks (weight alignment aside)
  size_t lds = 0;
  int64_t dim_res = 0;
  size_t res_off = 0, term_off = 0;  // within the device blob
};

}  // namespace

struct segpoly_fctp {
  std::vector<Irrep> in1, in2, out;
  std::vector<int64_t> off1, off2, offo;
  struct Path {
    int i, j, o;
    int64_t w_off;
  };
  std::vector<Path> paths;
  std::vector<double> alpha;
  int layout = 0, dtype = 0;
  unsigned flags = 0;
  int64_t dim1 = 0, dim2 = 0, dimo = 0, numel = 0;
  FcPass pass[3];                 // forward, input-1 gradient, input-2 gradient
  std::vector<FcDwPath> dw;
  int dw_nt = 1;                  // entry class of the weight-gradient launch
  bool dw_dma = false;            // weight-gradient staging straight into LDS
  size_t dw_lds = 0, dw_off = 0, ent_off = 0, tr_off = 0;
  std::vector<FcTrPath> tr_paths;     // segments of the weight transposition
  std::vector<FcEnt> ents;
  // the graph convolution form (per-edge weights); conv_error is why it is
  // unavailable for this descriptor ("" if available)
  std::string conv_error;
  std::vector<FcvBlock> cv_blocks;
  std::vector<FcvPath> cv_paths;
  std::vector<FcvQK> cv_qks;
  std::vector<FcvEnt> cv_ents;
  std::vector<FcvTile> cv_tiles;
  std::vector<FcvUT> cv_uts;
  std::vector<FcvQ> cv_qs;
  std::vector<FcvChunk> cv_chunks;
  std::vector<FcvBPath> cv_bpaths;    // backward: every path with its global rows
  std::string conv_bwd_error;         // why the backward is unavailable ("" if available)
  size_t cv_bwd_lds = 0;
  int cv_ncomp = 0, cv_max_nqk = 0, cv_lane_bits = 0, cv_n_ut = 1;
  size_t cv_lds = 0;
  size_t cv_off[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};  // blocks, paths, qks, ents, tiles, qs, chunks, bpaths, uts in the blob
  // one weight row per sample: tiles, paths, entry lists, entries
  std::vector<PsTile> ps_tiles;
  std::vector<PsPath> ps_paths;
  std::vector<PsList> ps_lists;
  std::vector<PsEnt> ps_ents;
  int ps_max_d = 1;
  size_t ps_off[4] = {0, 0, 0, 0};
  std::vector<unsigned char> blob;
  std::map<int, DeviceBuffer> dev;
  std::mutex mu;
};

namespace {

size_t elt(int dtype) { return dtype == SEGPOLY_F32 ? 4 : 8; }

// Entries of one term for result components 0..dr-1: coupling C[a, b, k]
// of the path seen with the result index `which` (0: a, 1: b, 2: k) and the
// other two as (P component, Q component).  Returns T, appends T * dr
// entries (zero-padded) to `ents`.
int add_entries(std::vector<FcEnt>& ents, const std::vector<double>& C, int d1, int d2, int d3, int which,
                double scale) {
  const int dr = which == 0 ? d1 : (which == 1 ? d2 : d3);
  std::vector<std::vector<FcEnt>> per(dr);
  for (int a = 0; a < d1; ++a)
    for (int b = 0; b < d2; ++b)
      for (int k = 0; k < d3; ++k) {
        const double c = C[(static_cast<size_t>(a) * d2 + b) * d3 + k];
        if (std::fabs(c) < 1e-13) continue;
        if (which == 0) per[a].push_back({b, k, scale * c});
        else if (which == 1) per[b].push_back({a, k, scale * c});
        else per[k].push_back({a, b, scale * c});
      }
  int T = 1;
  for (const auto& v : per) T = std::max<int>(T, static_cast<int>(v.size()));
  if (T > kFcMaxT) return -1;
  for (const auto& v : per)
    for (int e = 0; e < T; ++e) ents.push_back(e < static_cast<int>(v.size()) ? v[e] : FcEnt{0, 0, 0.0});
  return T;
}

// Samples per tile of result block R: whole samples, at most 128 rows,
// LDS within the limit (rows 128, else 64, 32, 16).
int pick_ts(int d, size_t per_sample, size_t budget) {
  for (int rows : {kFcRowsMax, 64, 32, 16}) {
    const int ts = std::max(1, rows / d);
    if (static_cast<size_t>(ts) * per_sample <= budget) return ts;
  }
  const size_t ts = per_sample ? budget / per_sample : 1;
  return ts >= 1 ? static_cast<int>(std::min<size_t>(ts, 16)) : 0;
}

int tn_for(int m) { return m <= 32 ? 32 : 64; }

size_t static_b_bytes(int tn, int dtype) {
  const int stride = tn + 16;
  return 2ull * 32 * stride * elt(dtype);
}

// Build pass `which` (0 forward, 1 dx1, 2 dx2).
int build_pass(segpoly_fctp* h, int which) {
  FcPass& P = h->pass[which];
  const std::vector<Irrep>& rb = which == 0 ? h->out : (which == 1 ? h->in1 : h->in2);
  const std::vector<int64_t>& roff = which == 0 ? h->offo : (which == 1 ? h->off1 : h->off2);
  if (rb.size() > static_cast<size_t>(kFcMaxRes))
    return fail(SEGPOLY_E_UNSUPPORTED, "more than 32 irreps blocks on one side");
  P.dim_res = roff.back();
  int mmax = 1;
  for (const auto& b : rb) mmax = std::max(mmax, b.mul);
  P.tn = tn_for(mmax);
  const size_t budget = product_lds_limit(h->dtype, P.tn) - static_b_bytes(P.tn, h->dtype);
  for (size_t r = 0; r < rb.size(); ++r) {
    FcRes R{};
    R.off = roff[r];
    R.d = 2 * rb[r].l + 1;
    R.m = rb[r].mul;
    R.term_begin = static_cast<int>(P.terms.size());
    size_t per_sample = 0;
    for (const auto& pa : h->paths) {
      const int blk = which == 0 ? pa.o : (which == 1 ? pa.i : pa.j);
      if (blk != static_cast<int>(r)) continue;
      const Irrep &a = h->in1[pa.i], &b = h->in2[pa.j], &o = h->out[pa.o];
      const int d1 = 2 * a.l + 1, d2 = 2 * b.l + 1, d3 = 2 * o.l + 1;
      const int64_t m1 = a.mul, m2 = b.mul, m3 = o.mul;
      FcTerm t{};
      t.w_off = pa.w_off;
      if (which == 0) {  // P = x1 (a, u), Q = x2 (b, v), result (k, w)
        t.p_op = 0, t.q_op = 1;
        t.p_d = d1, t.p_m = a.mul, t.p_off = h->off1[pa.i];
        t.q_d = d2, t.q_m = b.mul, t.q_off = h->off2[pa.j];
        t.s_p = m2 * m3, t.s_q = m3, t.s_r = 1;
      } else if (which == 1) {  // P = x2 (b, v), Q = g (k, w), result (a, u); weights W1[v][w][u]
        t.p_op = 1, t.q_op = 2;
        t.p_d = d2, t.p_m = b.mul, t.p_off = h->off2[pa.j];
        t.q_d = d3, t.q_m = o.mul, t.q_off = h->offo[pa.o];
        t.s_p = m3 * m1, t.s_q = m1, t.s_r = 1;
      } else {  // P = x1 (a, u), Q = g (k, w), result (b, v); weights W2[u][w][v]
        t.p_op = 0, t.q_op = 2;
        t.p_d = d1, t.p_m = a.mul, t.p_off = h->off1[pa.i];
        t.q_d = d3, t.q_m = o.mul, t.q_off = h->offo[pa.o];
        t.s_p = m3 * m2, t.s_q = m2, t.s_r = 1;
      }
      if (static_cast<int64_t>(t.p_m) * t.q_m >= (1ll << 31))
        return fail(SEGPOLY_E_UNSUPPORTED, "multiplicities too large (mul1 * mul2 must stay below 2^31)");
      t.ent = static_cast<int>(h->ents.size());
      const int which_idx = which == 0 ? 2 : (which == 1 ? 0 : 1);
      t.T = add_entries(h->ents, real_cg(a.l, b.l, o.l), d1, d2, d3, which_idx, h->alpha[pa.o]);
      if (t.T < 0) return fail(SEGPOLY_E_UNSUPPORTED, "more than 16 couplings per component in one path");
      if (t.p_m > t.q_m) {  // Q, held in registers along K, is the side with more channels
        std::swap(t.p_op, t.q_op);
        std::swap(t.p_d, t.q_d);
        std::swap(t.p_m, t.q_m);
        std::swap(t.p_off, t.q_off);
        std::swap(t.s_p, t.s_q);
        for (size_t e = t.ent; e < h->ents.size(); ++e) std::swap(h->ents[e].pa, h->ents[e].qb);
      }
      P.nt = std::max(P.nt, fc_t_class(t.T));
      per_sample = std::max(per_sample, static_cast<size_t>(fc_sample_stride(t.p_d, t.p_m)) * elt(h->dtype));
      P.terms.push_back(t);
    }
    R.term_end = static_cast<int>(P.terms.size());
    R.ts = pick_ts(R.d, per_sample, budget);
    if (R.ts < 1) return fail(SEGPOLY_E_UNSUPPORTED, "operand blocks too wide for the LDS of one workgroup");
    R.col_tiles = (R.m + P.tn - 1) / P.tn;
    if (R.m == 0) R.col_tiles = 0;
    P.lds = std::max(P.lds, static_cast<size_t>(R.ts) * per_sample);
    P.res.push_back(R);
  }
  // LDS-direct weight chunks: float, 32-column tiles, result blocks of whole
  // column tiles, and every term with the result channel the contiguous
  // weight index, whole 32-channel windows of Q, rows of a multiple of four
  // elements, at most four couplings per component (32-row chunks)
  P.lds_direct = h->dtype == SEGPOLY_F32 && P.tn == 32 && P.nt <= 4 && !P.terms.empty();
  for (const auto& R : P.res)
    if (R.m % 32) P.lds_direct = false;
  for (const auto& t : P.terms)
    if (t.s_r != 1 || t.q_m % 32 || t.w_off % 4 || t.s_q % 4 || t.s_p % 4) P.lds_direct = false;
  return SEGPOLY_OK;
}

int build_dw(segpoly_fctp* h) {
  if (h->paths.size() > static_cast<size_t>(kFcMaxPaths)) return fail(SEGPOLY_E_UNSUPPORTED, "more than 64 paths");
  for (const auto& pa : h->paths) {
    const Irrep &a = h->in1[pa.i], &b = h->in2[pa.j], &o = h->out[pa.o];
    const int d1 = 2 * a.l + 1, d2 = 2 * b.l + 1, d3 = 2 * o.l + 1;
    FcDwPath q{};
    q.p_op = 0, q.q_op = 1;
    q.p_d = d1, q.p_m = a.mul, q.q_d = d2, q.q_m = b.mul, q.g_d = d3, q.g_m = o.mul;
    q.p_off = h->off1[pa.i], q.q_off = h->off2[pa.j], q.g_off = h->offo[pa.o], q.w_off = pa.w_off;
    q.s_p = static_cast<int64_t>(b.mul) * o.mul, q.s_q = o.mul;
    q.ent = static_cast<int>(h->ents.size());
    q.T = add_entries(h->ents, real_cg(a.l, b.l, o.l), d1, d2, d3, 2, h->alpha[pa.o]);
    if (q.T < 0) return fail(SEGPOLY_E_UNSUPPORTED, "more than 16 couplings per component in one path");
    if (q.p_m > q.q_m) {  // Q, the 32-channel side of a tile, has more channels
      std::swap(q.p_op, q.q_op);
      std::swap(q.p_d, q.q_d);
      std::swap(q.p_m, q.q_m);
      std::swap(q.p_off, q.q_off);
      std::swap(q.s_p, q.s_q);
      for (size_t e = q.ent; e < h->ents.size(); ++e) std::swap(h->ents[e].pa, h->ents[e].qb);
    }
    const size_t per = (static_cast<size_t>(fc_sample_stride(q.p_d, q.p_m)) + fc_sample_stride(q.q_d, q.q_m) +
                        fc_sample_stride(q.g_d, q.g_m)) * elt(h->dtype);
    int ts = static_cast<int>(std::min<size_t>(kFcDwSamples, kLdsLimit / per)) & ~3;
    if (ts < 4) return fail(SEGPOLY_E_UNSUPPORTED, "operand blocks too wide for the weight-gradient kernel");
    q.ts = ts;
    h->dw_nt = std::max(h->dw_nt, fc_t_class(q.T));
    q.u_tiles = (q.p_m + kFcDwU - 1) / kFcDwU;
    q.v_tiles = (q.q_m + kFcDwV - 1) / kFcDwV;
    q.col_tiles = (q.g_m + kFcDwCols - 1) / kFcDwCols;
    h->dw_lds = std::max(h->dw_lds, static_cast<size_t>(ts) * per);
    h->dw.push_back(q);
  }
  // Paths whose output block has more components dispatch first: their
  // workgroups do proportionally more work, and starting them early keeps
  // the launch's tail short.
  std::stable_sort(h->dw.begin(), h->dw.end(), [](const FcDwPath& x, const FcDwPath& y) { return x.g_d > y.g_d; });
  // Float launches stage through the LDS-direct buffers when every staged
  // sample fits the per-lane copies and four samples of the three blocks
  // fit one buffer.
  bool dma = h->dtype == SEGPOLY_F32;
  for (const auto& q : h->dw) {
    const int ps = fc_sample_stride(q.p_d, q.p_m), qs = fc_sample_stride(q.q_d, q.q_m),
              gs = fc_sample_stride(q.g_d, q.g_m);
    dma = dma && std::max({ps, qs, gs}) <= 64 * kFcDwDmaJ && kFcDwDmaElems / (ps + qs + gs) >= 4;
  }
  if (dma) {
    for (auto& q : h->dw) {
      const int per = fc_sample_stride(q.p_d, q.p_m) + fc_sample_stride(q.q_d, q.q_m) +
                      fc_sample_stride(q.g_d, q.g_m);
      q.ts = std::min(kFcDwSamples, kFcDwDmaElems / per) & ~3;
    }
    h->dw_lds = 0;
  }
  h->dw_dma = dma;
  return SEGPOLY_OK;
}

// Tables of the convolution form: input 2 must be the edge harmonics (one
// channel per block).  Input-1 blocks of more than 64 channels are taken
// 64 channels (one u tile) at a time.
void build_conv(segpoly_fctp* h) {
  for (const auto& b : h->in2)
    if (b.mul != 1) {
      h->conv_error = "the convolution form needs one channel per input-2 block (edge harmonics)";
      return;
    }
  int mmax = 1;
  for (const auto& b : h->in1) mmax = std::max(mmax, b.mul);
  const int n_ut = (mmax + kFcvUTile - 1) / kFcvUTile;
  h->cv_n_ut = n_ut;
  int comp = 0;
  for (size_t i = 0; i < h->in1.size(); ++i) {
    const Irrep& b = h->in1[i];
    h->cv_blocks.push_back({h->off1[i], 2 * b.l + 1, b.mul, comp});
    comp += 2 * b.l + 1;
  }
  h->cv_ncomp = comp;
  int nwmax = 1;
  for (size_t o = 0; o < h->out.size(); ++o) {
    const Irrep& ob = h->out[o];
    const int d3 = 2 * ob.l + 1;
    if (ob.mul == 0) continue;
    const int path_begin = static_cast<int>(h->cv_paths.size());
    const int qk_begin = static_cast<int>(h->cv_qks.size());
    int nqk = 0;
    for (const auto& pa : h->paths) {
      if (pa.o != static_cast<int>(o)) continue;
      const Irrep &a = h->in1[pa.i], &b = h->in2[pa.j];
      const int d1 = 2 * a.l + 1, d2 = 2 * b.l + 1;
      h->cv_paths.push_back({pa.w_off, a.mul, nqk});
      const std::vector<double>& C = real_cg(a.l, b.l, ob.l);
      for (int k = 0; k < d3; ++k) {
        FcvQK q{static_cast<int>(h->cv_ents.size()), 0};
        for (int ia = 0; ia < d1; ++ia)
          for (int ib = 0; ib < d2; ++ib) {
            const double c = C[(static_cast<size_t>(ia) * d2 + ib) * d3 + k];
            if (std::fabs(c) < 1e-13) continue;
            h->cv_ents.push_back({h->cv_blocks[pa.i].comp + ia, static_cast<int>(h->off2[pa.j]) + ib,
                                  h->alpha[o] * c});
          }
        q.ent_end = static_cast<int>(h->cv_ents.size());
        h->cv_qks.push_back(q);
      }
      nqk += d3;
    }
    const int path_end = static_cast<int>(h->cv_paths.size());
    h->cv_max_nqk = std::max(h->cv_max_nqk, nqk);
    // per u tile: the full 16-channel chunks of every path inside it, then
    // the remaining channels one by one (u tiles start at multiples of 64,
    // so chunks never straddle two)
    const int ut_begin = static_cast<int>(h->cv_uts.size());
    for (int ut = 0; ut < n_ut; ++ut) {
      FcvUT U{static_cast<int>(h->cv_chunks.size()), 0, static_cast<int>(h->cv_qs.size()), 0};
      for (int pi = path_begin; pi < path_end; ++pi) {
        const FcvPath& P = h->cv_paths[pi];
        const int lo = ut * kFcvUTile, hi = std::min(P.m1, lo + kFcvUTile);
        int u = lo;
        for (; u + kFcvChunkU <= hi; u += kFcvChunkU)
          h->cv_chunks.push_back({P.w_off + static_cast<int64_t>(u) * ob.mul, P.qk, u});
        for (; u < hi; ++u) h->cv_qs.push_back({P.w_off + static_cast<int64_t>(u) * ob.mul, P.qk, u});
      }
      U.n_chunks = static_cast<int>(h->cv_chunks.size()) - U.chunk_begin;
      U.nq = static_cast<int>(h->cv_qs.size()) - U.q_begin;
      h->cv_uts.push_back(U);
    }
    for (int pi = path_begin; pi < path_end; ++pi) {
      const FcvPath& P = h->cv_paths[pi];
      h->cv_bpaths.push_back({P.w_off, h->offo[o], P.m1, ob.mul, d3, qk_begin + P.qk});
    }
    for (int w0 = 0; w0 < ob.mul; w0 += 64) {
      FcvTile t{};
      t.out_off = h->offo[o];
      t.d = d3, t.m = ob.mul, t.w0 = w0, t.nw = std::min(64, ob.mul - w0);
      t.path_begin = path_begin, t.path_end = path_end;
      t.qk_begin = qk_begin, t.nqk = nqk;
      t.ut_begin = ut_begin;
      nwmax = std::max(nwmax, t.nw);
      h->cv_tiles.push_back(t);
    }
  }
  int lanes = 1;
  while (lanes < std::max(std::min(mmax, kFcvUTile), nwmax)) lanes <<= 1;
  int bits = 0;
  while ((1 << bits) < lanes) ++bits;
  h->cv_lane_bits = bits;
  const size_t S = 64 >> bits;
  h->cv_lds = S * (static_cast<size_t>(h->cv_ncomp) * lanes + 1 + static_cast<size_t>(h->dim2) + 1 +
                   static_cast<size_t>(h->cv_max_nqk) * lanes + 1) * elt(h->dtype);
  if (h->cv_lds > 64 * 1024) {
    h->conv_error = "the convolution form's per-edge rows exceed the LDS of one wave";
    return;
  }
  const size_t nrows = h->cv_qks.size();
  h->cv_bwd_lds = (S * (2 * (static_cast<size_t>(h->cv_ncomp) * lanes + 1) + static_cast<size_t>(h->dim2) + 1 +
                        2 * (nrows * lanes + 1) + static_cast<size_t>(h->dim2) * lanes + 1) +
                   static_cast<size_t>(h->dimo)) * elt(h->dtype);
  if (h->cv_bwd_lds > 64 * 1024) h->conv_bwd_error = "the convolution backward's per-edge rows exceed the LDS of one wave";
}

// Tables of the per-sample form: paths grouped by output block, each with
// its coupling entries listed three ways (by output, input-1 and input-2
// component); tiles of up to 64 output channels.
void build_ps(segpoly_fctp* h) {
  for (size_t o = 0; o < h->out.size(); ++o) {
    const Irrep& ob = h->out[o];
    const int d3 = 2 * ob.l + 1;
    const int path_begin = static_cast<int>(h->ps_paths.size());
    for (const auto& pa : h->paths) {
      if (pa.o != static_cast<int>(o)) continue;
      const Irrep &a = h->in1[pa.i], &b = h->in2[pa.j];
      if (a.mul == 0 || b.mul == 0) continue;  // no (u, v) pairs, no weights
      const int d1 = 2 * a.l + 1, d2 = 2 * b.l + 1;
      const std::vector<double>& C = real_cg(a.l, b.l, ob.l);
      std::vector<PsEnt> nz;
      for (int ia = 0; ia < d1; ++ia)
        for (int ib = 0; ib < d2; ++ib)
          for (int k = 0; k < d3; ++k) {
            const double c = C[(static_cast<size_t>(ia) * d2 + ib) * d3 + k];
            if (std::fabs(c) >= 1e-13) nz.push_back({ia, ib, k, 0, h->alpha[o] * c});
          }
      PsPath P{};
      P.woff = pa.w_off;
      P.off1 = static_cast<int>(h->off1[pa.i]);
      P.off2 = static_cast<int>(h->off2[pa.j]);
      P.m1 = a.mul, P.m2 = b.mul, P.d1 = d1, P.d2 = d2;
      // which = 0: by output component, 1: by input-1, 2: by input-2
      auto lists = [&](int which, int count) {
        const int first = static_cast<int>(h->ps_lists.size());
        for (int q = 0; q < count; ++q) {
          PsList L{static_cast<int>(h->ps_ents.size()), 0};
          for (const PsEnt& e : nz)
            if ((which == 0 ? e.k : which == 1 ? e.a : e.b) == q) h->ps_ents.push_back(e);
          L.end = static_cast<int>(h->ps_ents.size());
          h->ps_lists.push_back(L);
        }
        return first;
      };
      P.k_list = lists(0, d3);
      P.a_list = lists(1, d1);
      P.b_list = lists(2, d2);
      h->ps_paths.push_back(P);
    }
    const int path_end = static_cast<int>(h->ps_paths.size());
    for (int w0 = 0; w0 < ob.mul; w0 += 64) {
      PsTile t{};
      t.offo = static_cast<int>(h->offo[o]);
      t.d3 = d3, t.m3 = ob.mul, t.w0 = w0, t.nw = std::min(64, ob.mul - w0);
      t.path_begin = path_begin, t.path_end = path_end;
      while ((1 << t.lane_bits) < t.nw) ++t.lane_bits;
      h->ps_max_d = std::max(h->ps_max_d, d3);
      h->ps_tiles.push_back(t);
    }
  }
}

template <typename V>
size_t append(std::vector<unsigned char>& blob, const std::vector<V>& v) {
  const size_t off = (blob.size() + 255) & ~size_t(255);
  blob.resize(off + v.size() * sizeof(V));
  if (!v.empty()) std::memcpy(blob.data() + off, v.data(), v.size() * sizeof(V));
  return off;
}

// Per-call tile map of pass `which` for n samples; false if the grid would
// not fit.
bool fill_tiles(const FcPass& P, int64_t n, FcTiles& t) {
  t.n_res = static_cast<int>(P.res.size());
  int64_t acc = 0;
  for (int r = 0; r < t.n_res; ++r) {
    t.tile_begin[r] = static_cast<int>(acc);
    const FcRes& R = P.res[r];
    acc += (n + R.ts - 1) / R.ts * R.col_tiles;
    if (acc >= kMaxGridX) return false;
  }
  t.tile_begin[t.n_res] = static_cast<int>(acc);
  return true;
}

bool fill_dw_tiles(const segpoly_fctp* h, int64_t n, FcDwTiles& t) {
  t.n_paths = static_cast<int>(h->dw.size());
  const int64_t chunks = (n + kFcDwChunk - 1) / kFcDwChunk;
  t.chunks = static_cast<int>(chunks);
  int64_t acc = 0;
  for (int p = 0; p < t.n_paths; ++p) {
    t.tile_begin[p] = static_cast<int>(acc);
    acc += chunks * h->dw[p].u_tiles * h->dw[p].v_tiles * h->dw[p].col_tiles;
    if (acc >= kMaxGridX) return false;
  }
  t.tile_begin[t.n_paths] = static_cast<int>(acc);
  return true;
}

const unsigned char* device_blob(segpoly_fctp* h, int* st) {
  return static_cast<const unsigned char*>(upload(h->dev, h->mu, h->blob.data(), h->blob.size(), st));
}

int run_pass(segpoly_fctp* h, const unsigned char* db, int which, const void* x1, const void* x2, const void* g,
             const void* w, int64_t n, void* res, void* stream) {
  const FcPass& P = h->pass[which];
  FcTiles t{};
  if (!fill_tiles(P, n, t)) return fail(SEGPOLY_E_UNSUPPORTED, "too many samples for one launch");
  FcArgs a{};
  a.op[0] = x1, a.op[1] = x2, a.op[2] = g;
  a.dim[0] = h->dim1, a.dim[1] = h->dim2, a.dim[2] = h->dimo;
  a.w = w;
  a.res = res;
  a.dim_res = P.dim_res;
  a.n = n;
  a.res_tab = reinterpret_cast<const FcRes*>(db + P.res_off);
  a.terms = reinterpret_cast<const FcTerm*>(db + P.term_off);
  a.ents = reinterpret_cast<const FcEnt*>(db + h->ent_off);
  a.tn = P.tn;
  a.nt = P.nt;
  a.lds_direct = P.lds_direct && reinterpret_cast<uintptr_t>(w) % 16 == 0;
  a.lds_bytes = P.lds;
  a.dtype = h->dtype;
  a.layout = h->layout;
  a.stream = stream;
  const int rc = launch_fctp(a, t);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return SEGPOLY_OK;
}

size_t dw_workspace(const segpoly_fctp* h, int64_t n) {
  const int64_t chunks = (n + kFcDwChunk - 1) / kFcDwChunk;
  return static_cast<size_t>(round_up_256(chunks * h->numel * static_cast<int64_t>(elt(h->dtype))));
}

// bytes of one transposed weight copy (the input-gradient passes read two)
size_t tr_bytes(const segpoly_fctp* h) {
  return static_cast<size_t>(round_up_256(h->numel * static_cast<int64_t>(elt(h->dtype))));
}

// workspace of fctp_bwd: [dW partials][W1][W2]
size_t bwd_workspace(const segpoly_fctp* h, int64_t n) {
  return n > 0 && h->numel > 0 ? dw_workspace(h, n) + 2 * tr_bytes(h) : 0;
}

}  // namespace

extern "C" {

int fctp_create(const char* irreps_in1, const char* irreps_in2, const char* irreps_out, int layout, int dtype,
                unsigned flags, fctp_handle* out) {
  if (!out) return fail(SEGPOLY_E_INVALID, "null handle pointer");
  *out = nullptr;
  if (!irreps_in1 || !irreps_in2 || !irreps_out) return fail(SEGPOLY_E_INVALID, "null irreps string");
  if (layout != SEGPOLY_MUL_IR && layout != SEGPOLY_IR_MUL) return fail(SEGPOLY_E_INVALID, "bad layout");
  if (dtype != SEGPOLY_F32 && dtype != SEGPOLY_F64) return fail(SEGPOLY_E_INVALID, "bad dtype");
  if (flags & ~(SEGPOLY_VALIDATE | SEGPOLY_REDUCE_MEAN)) return fail(SEGPOLY_E_INVALID, "unknown flag bits");
  segpoly_fctp* h = nullptr;
  try {
    h = new segpoly_fctp();
    h->in1 = parse_any(irreps_in1);
    h->in2 = parse_any(irreps_in2);
    h->out = parse_any(irreps_out);
  } catch (const ParseError& e) {
    delete h;
    return fail(SEGPOLY_E_PARSE, e.what());
  } catch (const std::bad_alloc&) {
    delete h;
    return fail(SEGPOLY_E_OOM, "out of host memory");
  } catch (const std::exception& e) {
    delete h;
    return fail(SEGPOLY_E_PARSE, e.what());
  }
  int so3 = 0, o3 = 0;
  for (const auto* v : {&h->in1, &h->in2, &h->out})
    for (const auto& b : *v) {
      (b.p == 0 ? so3 : o3) = 1;
      if (b.l > kMaxL) {
        delete h;
        return fail(SEGPOLY_E_UNSUPPORTED, "l above 6");
      }
    }
  if (so3 && o3) {
    delete h;
    return fail(SEGPOLY_E_PARSE, "mixing SO(3) and O(3) irreps");
  }
  h->layout = layout;
  h->dtype = dtype;
  h->flags = flags;
  h->off1 = offsets(h->in1);
  h->off2 = offsets(h->in2);
  h->offo = offsets(h->out);
  h->dim1 = h->off1.back(), h->dim2 = h->off2.back(), h->dimo = h->offo.back();
  // paths in the order input-1 block, input-2 block, output block; one
  // weight segment of mul1 * mul2 * mul3 (w fastest) per path
  std::vector<int64_t> fan(h->out.size(), 0);
  int64_t woff = 0;
  for (size_t i = 0; i < h->in1.size(); ++i)
    for (size_t j = 0; j < h->in2.size(); ++j)
      for (size_t o = 0; o < h->out.size(); ++o) {
        const Irrep &a = h->in1[i], &b = h->in2[j], &c = h->out[o];
        if (c.l < std::abs(a.l - b.l) || c.l > a.l + b.l || c.p != a.p * b.p) continue;
        h->paths.push_back({static_cast<int>(i), static_cast<int>(j), static_cast<int>(o), woff});
        h->tr_paths.push_back({woff, a.mul, b.mul, c.mul});
        woff += static_cast<int64_t>(a.mul) * b.mul * c.mul;
        fan[o] += static_cast<int64_t>(a.mul) * b.mul;
      }
  h->numel = woff;
  for (size_t o = 0; o < h->out.size(); ++o) h->alpha.push_back(fan[o] ? 1.0 / std::sqrt(double(fan[o])) : 0.0);
  int rc = SEGPOLY_OK;
  try {
    for (int w = 0; w < 3 && rc == SEGPOLY_OK; ++w) rc = build_pass(h, w);
    if (rc == SEGPOLY_OK) rc = build_dw(h);
    if (rc == SEGPOLY_OK) build_conv(h);
    if (rc == SEGPOLY_OK) build_ps(h);
    if (rc == SEGPOLY_OK) {
      for (int w = 0; w < 3; ++w) {
        h->pass[w].res_off = append(h->blob, h->pass[w].res);
        h->pass[w].term_off = append(h->blob, h->pass[w].terms);
      }
      h->dw_off = append(h->blob, h->dw);
      h->tr_off = append(h->blob, h->tr_paths);
      h->ent_off = append(h->blob, h->ents);
      h->cv_off[0] = append(h->blob, h->cv_blocks);
      h->cv_off[1] = append(h->blob, h->cv_paths);
      h->cv_off[2] = append(h->blob, h->cv_qks);
      h->cv_off[3] = append(h->blob, h->cv_ents);
      h->cv_off[4] = append(h->blob, h->cv_tiles);
      h->cv_off[5] = append(h->blob, h->cv_qs);
      h->cv_off[6] = append(h->blob, h->cv_chunks);
      h->cv_off[7] = append(h->blob, h->cv_bpaths);
      h->cv_off[8] = append(h->blob, h->cv_uts);
      h->ps_off[0] = append(h->blob, h->ps_tiles);
      h->ps_off[1] = append(h->blob, h->ps_paths);
      h->ps_off[2] = append(h->blob, h->ps_lists);
      h->ps_off[3] = append(h->blob, h->ps_ents);
    }
  } catch (const std::bad_alloc&) {
    rc = fail(SEGPOLY_E_OOM, "out of host memory");
  }
  if (rc != SEGPOLY_OK) {
    delete h;
    return rc;
  }
  *out = h;
  return ok();
}

int fctp_query(fctp_handle h, int key, int64_t* value) {
  if (!h || !value) return fail(SEGPOLY_E_INVALID, "null argument");
  switch (key) {
    case SEGPOLY_Q_DIM_IN1: *value = h->dim1; break;
    case SEGPOLY_Q_DIM_IN2: *value = h->dim2; break;
    case SEGPOLY_Q_DIM_OUT: *value = h->dimo; break;
    case SEGPOLY_Q_WEIGHT_NUMEL: *value = h->numel; break;
    case SEGPOLY_Q_NUM_PATHS: *value = static_cast<int64_t>(h->paths.size()); break;
    default: return fail(SEGPOLY_E_INVALID, "unknown query key");
  }
  return ok();
}

int fctp_path_info(fctp_handle h, int p, int64_t* info4) {
  if (!h || !info4) return fail(SEGPOLY_E_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int>(h->paths.size())) return fail(SEGPOLY_E_INVALID, "path index out of range");
  info4[0] = h->paths[p].i;
  info4[1] = h->paths[p].j;
  info4[2] = h->paths[p].o;
  info4[3] = h->paths[p].w_off;
  return ok();
}

int fctp_fwd(fctp_handle h, const void* x1, const void* x2, const void* w, int64_t n, void* out, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative sample count");
  if (n == 0) return ok();
  if (!out || (h->numel > 0 && !w) || (h->dim1 > 0 && !x1) || (h->dim2 > 0 && !x2))
    return fail(SEGPOLY_E_INVALID, "null buffer");
  int st = SEGPOLY_OK;
  const unsigned char* db = device_blob(h, &st);
  if (!db) return st;
  const int rc = run_pass(h, db, 0, x1, x2, nullptr, w, n, out, stream);
  return rc ? rc : ok();
}

int fctp_bwd_workspace(fctp_handle h, int64_t n, size_t* bytes) {
  if (!h || !bytes) return fail(SEGPOLY_E_INVALID, "null argument");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative sample count");
  *bytes = bwd_workspace(h, n);
  return ok();
}

int fctp_bwd(fctp_handle h, const void* x1, const void* x2, const void* w, const void* grad_out, int64_t n,
             void* grad_x1, void* grad_x2, void* grad_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative sample count");
  const bool any = grad_x1 || grad_x2 || grad_w;
  if (any && workspace_bytes < bwd_workspace(h, n))
    return fail(SEGPOLY_E_INVALID, "workspace too small: need " + std::to_string(bwd_workspace(h, n)) + " bytes");
  if (any && bwd_workspace(h, n) > 0 && !workspace) return fail(SEGPOLY_E_INVALID, "null workspace");
  if (n > 0) {
    if ((h->dimo > 0 && !grad_out) || (h->dim1 > 0 && !x1 && (grad_x2 || grad_w)) ||
        (h->dim2 > 0 && !x2 && (grad_x1 || grad_w)) || (h->numel > 0 && !w && (grad_x1 || grad_x2)))
      return fail(SEGPOLY_E_INVALID, "null buffer");
  }
  if (n == 0) {
    if (grad_w && h->numel > 0) {
      const int rc = launch_fill_zero(grad_w, h->numel, h->dtype, stream);
      if (rc) return fail(SEGPOLY_E_HIP, std::string("fill: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
    }
    return ok();
  }
  int st = SEGPOLY_OK;
  const unsigned char* db = device_blob(h, &st);
  if (!db) return st;
  if ((grad_x1 || grad_x2) && h->numel > 0) {  // the transposed weights both input gradients read
    unsigned char* ws = static_cast<unsigned char*>(workspace) + dw_workspace(h, n);
    FcTrArgs a{};
    a.w = w;
    a.w1 = ws;
    a.w2 = ws + tr_bytes(h);
    a.paths = reinterpret_cast<const FcTrPath*>(db + h->tr_off);
    a.n_paths = static_cast<int>(h->tr_paths.size());
    a.numel = h->numel;
    a.dtype = h->dtype;
    a.stream = stream;
    const int rc = launch_fctp_transpose(a);
    if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp transpose: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  }
  const unsigned char* w1 = static_cast<const unsigned char*>(workspace) + dw_workspace(h, n);
  if (grad_x1) {
    const int rc = run_pass(h, db, 1, x1, x2, grad_out, h->numel > 0 ? w1 : w, n, grad_x1, stream);
    if (rc) return rc;
  }
  if (grad_x2) {
    const int rc = run_pass(h, db, 2, x1, x2, grad_out, h->numel > 0 ? w1 + tr_bytes(h) : w, n, grad_x2, stream);
    if (rc) return rc;
  }
  if (grad_w && h->numel > 0) {
    FcDwTiles t{};
    if (!fill_dw_tiles(h, n, t)) return fail(SEGPOLY_E_UNSUPPORTED, "too many samples for one launch");
    FcDwArgs a{};
    a.x1 = x1, a.x2 = x2, a.g = grad_out;
    a.dim1 = h->dim1, a.dim2 = h->dim2, a.dimo = h->dimo;
    a.part = workspace;
    a.dw = grad_w;
    a.numel = h->numel;
    a.n = n;
    a.paths = reinterpret_cast<const FcDwPath*>(db + h->dw_off);
    a.ents = reinterpret_cast<const FcEnt*>(db + h->ent_off);
    a.nt = h->dw_nt;
    a.lds_bytes = h->dw_lds;
    a.dma = h->dw_dma ? 1 : 0;
    a.dtype = h->dtype;
    a.layout = h->layout;
    a.stream = stream;
    const int rc = launch_fctp_dw(a, t);
    if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp dw launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  }
  return ok();
}

}  // extern "C"

namespace {

// Shared checks and arguments of the per-sample entry points; 0 or an error.
int ps_args(segpoly_fctp* h, int64_t n, bool bwd, FcPsArgs& a, const unsigned char** db) {
  const size_t e = elt(h->dtype);
  a.lds_bytes = bwd ? ps_lds_bwd(h->dim1, h->dim2, h->ps_max_d, e) : ps_lds_fwd(h->dim1, h->dim2, h->ps_max_d, e);
  if (a.lds_bytes > static_cast<size_t>(kPsLdsLimit))
    return fail(SEGPOLY_E_UNSUPPORTED, "one sample's staged rows exceed 64 KB of LDS");
  if (h->numel * static_cast<int64_t>(e) > 0x7fffffff)
    return fail(SEGPOLY_E_UNSUPPORTED, "a weight row of 2 GiB or more");
  if (n > kMaxGridX || (!bwd && h->ps_tiles.size() > 65535))
    return fail(SEGPOLY_E_UNSUPPORTED, "too many samples or tiles for one launch");
  int st = SEGPOLY_OK;
  *db = device_blob(h, &st);
  if (!*db) return st;
  a.n = n;
  a.dim1 = h->dim1, a.dim2 = h->dim2, a.dimo = h->dimo, a.numel = h->numel;
  a.tiles = reinterpret_cast<const PsTile*>(*db + h->ps_off[0]);
  a.paths = reinterpret_cast<const PsPath*>(*db + h->ps_off[1]);
  a.lists = reinterpret_cast<const PsList*>(*db + h->ps_off[2]);
  a.ents = reinterpret_cast<const PsEnt*>(*db + h->ps_off[3]);
  a.n_tiles = static_cast<int>(h->ps_tiles.size());
  a.max_d = h->ps_max_d;
  a.dtype = h->dtype;
  a.layout = h->layout;
  return SEGPOLY_OK;
}

}  // namespace

extern "C" {

int fctp_fwd_per_sample(fctp_handle h, const void* x1, const void* x2, const void* w, int64_t n, void* out,
                        void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative sample count");
  if (n == 0) return ok();
  if (!out || (h->numel > 0 && !w) || (h->dim1 > 0 && !x1) || (h->dim2 > 0 && !x2))
    return fail(SEGPOLY_E_INVALID, "null buffer");
  FcPsArgs a{};
  const unsigned char* db = nullptr;
  int rc = ps_args(h, n, false, a, &db);
  if (rc) return rc;
  a.x1 = x1, a.x2 = x2, a.w = w, a.out = out;
  a.stream = stream;
  rc = launch_fctp_ps_fwd(a);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp per-sample launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int fctp_bwd_per_sample(fctp_handle h, const void* x1, const void* x2, const void* w, const void* grad_out,
                        int64_t n, void* grad_x1, void* grad_x2, void* grad_w, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative sample count");
  if (n == 0 || !(grad_x1 || grad_x2 || grad_w)) return ok();
  if ((h->dimo > 0 && !grad_out) || (h->dim1 > 0 && !x1 && (grad_x2 || grad_w)) ||
      (h->dim2 > 0 && !x2 && (grad_x1 || grad_w)) || (h->numel > 0 && !w && (grad_x1 || grad_x2)))
    return fail(SEGPOLY_E_INVALID, "null buffer");
  FcPsArgs a{};
  const unsigned char* db = nullptr;
  int rc = ps_args(h, n, true, a, &db);
  if (rc) return rc;
  a.x1 = x1, a.x2 = x2, a.w = w, a.g = grad_out;
  a.dx1 = grad_x1, a.dx2 = grad_x2, a.dw = h->numel > 0 ? grad_w : nullptr;
  // 16-byte pieces of the weight rows: every output multiplicity (so every
  // row, segment and tile start) a multiple of 16 bytes, and aligned buffers
  const int64_t vw = 16 / static_cast<int64_t>(elt(h->dtype));
  bool vec = reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(a.dw) % 16 == 0;
  for (const auto& b : h->out) vec = vec && b.mul % vw == 0;
  a.vec = vec ? 1 : 0;
  a.stream = stream;
  rc = launch_fctp_ps_bwd(a);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp per-sample backward launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int fctp_conv_fwd(fctp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, int64_t w_rows,
                  const void* src, const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* out,
                  void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (!h->conv_error.empty()) return fail(SEGPOLY_E_UNSUPPORTED, h->conv_error);
  if (n_src < 0 || n_edges < 0 || n_nodes < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (w_rows != 1 && w_rows != n_edges) return fail(SEGPOLY_E_INVALID, "w_rows must be 1 (shared) or n_edges");
  if (n_nodes == 0) return ok();
  if (!out) return fail(SEGPOLY_E_INVALID, "null output");
  if (n_edges > 0 && (!src || !dst || (h->dim2 > 0 && !sh) || (h->numel > 0 && !w) || (n_src > 0 && !x)))
    return fail(SEGPOLY_E_INVALID, "null buffer");
  if (n_nodes > kMaxGridX) return fail(SEGPOLY_E_UNSUPPORTED, "too many destination rows for one launch");
  if (h->flags & SEGPOLY_VALIDATE) {
    const int st = idx_dtype == SEGPOLY_I32 ? check_indices<int32_t>(src, dst, n_edges, n_src, n_nodes, stream)
                                            : check_indices<int64_t>(src, dst, n_edges, n_src, n_nodes, stream);
    if (st) return st;
  }
  int st = SEGPOLY_OK;
  const unsigned char* db = device_blob(h, &st);
  if (!db) return st;
  FcvArgs a{};
  a.x = x, a.sh = sh, a.w = w, a.src = src, a.dst = dst;
  a.n_src = n_src, a.n_edges = n_edges, a.n_nodes = n_nodes;
  a.dim1 = h->dim1, a.dim2 = h->dim2, a.dimo = h->dimo;
  a.w_stride = w_rows == 1 && n_edges != 1 ? 0 : h->numel;
  a.out = out;
  a.mean = (h->flags & SEGPOLY_REDUCE_MEAN) ? 1 : 0;
  a.blocks = reinterpret_cast<const FcvBlock*>(db + h->cv_off[0]);
  a.paths = reinterpret_cast<const FcvPath*>(db + h->cv_off[1]);
  a.qks = reinterpret_cast<const FcvQK*>(db + h->cv_off[2]);
  a.ents = reinterpret_cast<const FcvEnt*>(db + h->cv_off[3]);
  a.tiles = reinterpret_cast<const FcvTile*>(db + h->cv_off[4]);
  a.qs = reinterpret_cast<const FcvQ*>(db + h->cv_off[5]);
  a.chunks = reinterpret_cast<const FcvChunk*>(db + h->cv_off[6]);
  a.n_blocks = static_cast<int>(h->cv_blocks.size());
  a.n_tiles = static_cast<int>(h->cv_tiles.size());
  a.ncomp = h->cv_ncomp;
  a.max_nqk = h->cv_max_nqk;
  a.lane_bits = h->cv_lane_bits;
  a.uts = reinterpret_cast<const FcvUT*>(db + h->cv_off[8]);
  a.n_ut = h->cv_n_ut;
  a.lds_bytes = h->cv_lds;
  a.dtype = h->dtype, a.layout = h->layout, a.idx = idx_dtype;
  a.stream = stream;
  const int rc = launch_fcconv(a);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp conv launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

// Per-edge messages [n_edges][dim1]; with one shared weight row then,
// 256-byte aligned, the per-edge weight gradients [n_edges][numel] and,
// aligned again, their partial sums [ceil(n_edges / kTpDwChunk)][numel].
static size_t fcv_bwd_ws(const segpoly_fctp* h, int64_t n_edges, bool shared, int64_t* dw_off) {
  const int64_t esz = static_cast<int64_t>(elt(h->dtype));
  int64_t b = round_up_256(n_edges * h->dim1 * esz);
  if (shared && n_edges > 0 && h->numel > 0) {
    if (dw_off) *dw_off = b;
    const int64_t chunks = (n_edges + kTpDwChunk - 1) / kTpDwChunk;
    b += round_up_256(n_edges * h->numel * esz) + chunks * h->numel * esz;
  }
  return static_cast<size_t>(b);
}

int fctp_conv_bwd_workspace(fctp_handle h, int64_t n_edges, int64_t w_rows, size_t* bytes) {
  if (!h || !bytes) return fail(SEGPOLY_E_INVALID, "null argument");
  if (n_edges < 0) return fail(SEGPOLY_E_INVALID, "negative edge count");
  if (w_rows != 1 && w_rows != n_edges) return fail(SEGPOLY_E_INVALID, "w_rows must be 1 (shared) or n_edges");
  *bytes = fcv_bwd_ws(h, n_edges, w_rows == 1 && n_edges != 1, nullptr);
  return ok();
}

int fctp_conv_bwd(fctp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, int64_t w_rows,
                  const void* src, const void* dst, const void* src_perm, int idx_dtype, int64_t n_edges,
                  int64_t n_nodes, const void* grad_out, void* grad_x, void* grad_sh, void* grad_w, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (!h->conv_error.empty()) return fail(SEGPOLY_E_UNSUPPORTED, h->conv_error);
  if (!h->conv_bwd_error.empty()) return fail(SEGPOLY_E_UNSUPPORTED, h->conv_bwd_error);
  if (n_src < 0 || n_edges < 0 || n_nodes < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (w_rows != 1 && w_rows != n_edges) return fail(SEGPOLY_E_INVALID, "w_rows must be 1 (shared) or n_edges");
  const bool shared = w_rows == 1 && n_edges != 1;
  int64_t dw_off = 0;
  const size_t need = fcv_bwd_ws(h, n_edges, shared, &dw_off);
  if (workspace_bytes < need) return fail(SEGPOLY_E_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((n_src > 0 && !grad_x) || (n_edges > 0 && (!grad_sh || !grad_w)) || (shared && h->numel > 0 && !grad_w))
    return fail(SEGPOLY_E_INVALID, "null gradient buffer");
  if (n_edges > 0 && (!src || !dst || !src_perm || !workspace || (h->dim2 > 0 && !sh) || (h->numel > 0 && !w) ||
                      (n_src > 0 && !x) || (n_nodes > 0 && h->dimo > 0 && !grad_out)))
    return fail(SEGPOLY_E_INVALID, "null buffer");
  if (n_nodes > kMaxGridX || n_src > kMaxGridX) return fail(SEGPOLY_E_UNSUPPORTED, "too many rows for one launch");
  if (n_edges == 0) {  // dx = 0 (and a shared weight gradient)
    int rc = launch_fill_zero(grad_x, n_src * h->dim1, h->dtype, stream);
    if (!rc && shared) rc = launch_fill_zero(grad_w, h->numel, h->dtype, stream);
    if (rc) return fail(SEGPOLY_E_HIP, std::string("fill: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
    return ok();
  }
  if (h->flags & SEGPOLY_VALIDATE) {
    int st = idx_dtype == SEGPOLY_I32 ? check_indices<int32_t>(src, dst, n_edges, n_src, n_nodes, stream)
                                      : check_indices<int64_t>(src, dst, n_edges, n_src, n_nodes, stream);
    if (st) return st;
    st = idx_dtype == SEGPOLY_I32 ? check_perm<int32_t>(src, src_perm, n_edges, stream)
                                  : check_perm<int64_t>(src, src_perm, n_edges, stream);
    if (st) return st;
  }
  int st = SEGPOLY_OK;
  const unsigned char* db = device_blob(h, &st);
  if (!db) return st;
  FcvBwdArgs a{};
  a.x = x, a.sh = sh, a.w = w, a.g = grad_out, a.src = src, a.dst = dst, a.perm = src_perm;
  a.n_src = n_src, a.n_edges = n_edges, a.n_nodes = n_nodes;
  a.dim1 = h->dim1, a.dim2 = h->dim2, a.dimo = h->dimo, a.numel = h->numel;
  a.mean = (h->flags & SEGPOLY_REDUCE_MEAN) ? 1 : 0;
  a.dx = grad_x, a.dsh = grad_sh, a.dw = grad_w, a.msg = workspace;
  a.shared_w = shared ? 1 : 0;
  a.dw_ws_off = dw_off;
  a.blocks = reinterpret_cast<const FcvBlock*>(db + h->cv_off[0]);
  a.qks = reinterpret_cast<const FcvQK*>(db + h->cv_off[2]);
  a.ents = reinterpret_cast<const FcvEnt*>(db + h->cv_off[3]);
  a.bpaths = reinterpret_cast<const FcvBPath*>(db + h->cv_off[7]);
  a.n_blocks = static_cast<int>(h->cv_blocks.size());
  a.n_bpaths = static_cast<int>(h->cv_bpaths.size());
  a.nrows = static_cast<int>(h->cv_qks.size());
  a.ncomp = h->cv_ncomp;
  a.lane_bits = h->cv_lane_bits;
  a.n_ut = h->cv_n_ut;
  a.lds_bytes = h->cv_bwd_lds;
  a.dtype = h->dtype, a.layout = h->layout, a.idx = idx_dtype;
  a.stream = stream;
  const int rc = launch_fcconv_bwd(a);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("fctp conv backward launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int fctp_destroy(fctp_handle h) {
  if (!h) return ok();
  free_all(h->dev);
  delete h;
  return ok();
}

}  // extern "C"
