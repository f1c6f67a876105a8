// Decode path launcher: three launches per layer (or per set of given routes).
//
//   1. router logits (when routing is fused), x quantized for the gate/up
//      rows, and (more than one token, VQ formats) the shared expert's
//      gate/up + SwiGLU;
//   2. exact top-k, routed gate/up + SwiGLU, routed h quantized in groups of
//      16, and (one token) the shared expert's gate/up + SwiGLU, which
//      streams while the blocks wait for the router logits and the top-k;
//   3. routed and shared down projections and the fixed-order combine.
//
// With several tokens (block formats) a planning launch between 1 and 2
// takes the top-k and lists the distinct experts in one block while its
// other blocks run the tokens' shared gate/up (and, with the caller's
// routes, quantize x, so that launch 1 is not needed), and 2 and 3 run over
// those experts (decode_unique.hip, decode_plan.hpp).
//
// The kernels are in decode_k1/k2/k3.hip; their common pieces (activation
// fixed point, IQ2 nibble table, weight pieces, dot products) in
// decode_common.hpp.
#include "decode_common.hpp"

namespace qmoe {
namespace dec {
hipError_t launch_k1(const DecodeArgs& a, const K1Plan& pl, int fmt_s, int gu_layout, hipStream_t s);
hipError_t launch_k2(const DecodeArgs& a, int fmt, int fs, int gcnt, int blocks, int down_layout, hipStream_t s);
hipError_t launch_k3(const DecodeArgs& a, int fmt_down, int fmt_shared, hipStream_t s);
hipError_t launch_plan(const DecodeArgs& a, hipStream_t s);
hipError_t launch_plan_shared(const DecodeArgs& a, const K1Plan& pl, int fmt_s, int gu_layout, hipStream_t s);
hipError_t launch_k3u(const DecodeArgs& a, int fmt_down, int fmt_shared, hipStream_t s);
}  // namespace dec

using namespace dec;

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecodeWsLayout {
  size_t xq, xs, xq_s, xs_s, hsh, hq, hs, hf, plan, total;
};

DecodeWsLayout ws_layout(int T, int k, int d, int f) {
  DecodeWsLayout L;
  size_t off = 0;
  L.xq = off;
  off = align256(off + (size_t)T * (d / 64) * CHUNK_BYTES);
  L.xs = off;
  off = align256(off + (size_t)T * (d / 64) * 4);
  L.xq_s = off;
  off = align256(off + (size_t)T * (d / 64) * CHUNK_BYTES);
  L.xs_s = off;
  off = align256(off + (size_t)T * (d / 64) * 4);
  L.hsh = off;
  off = align256(off + (size_t)T * f * 4);
  L.hq = off;
  off = align256(off + (size_t)T * k * (f / 16) * G16_BYTES);
  L.hs = off;
  off = align256(off + (size_t)T * k * (f / 16) * 4);
  L.hf = off;
  off = align256(off + (size_t)T * k * f * 4);
  L.plan = off;  // distinct experts (at most T k) and the routes grouped by them
  off = align256(off + (size_t)(2 + 3 * T * k) * 4);
  L.total = off;
  return L;
}

// Groups of 16 routed h rows per gate/up block: GCNT minimises (rounds of
// blocks) x (work per block), blocks never straddling a token.  Several
// tokens of the block formats (wide6) take blocks of 6 groups once those make
// at least two rounds of the GPU: fewer, longer blocks (measured 6 % faster
// at 8 tokens, 4 % at 4; at 2 tokens, one round, slower).
int gcnt_of(int k, int f, int T, int ncu, bool wide6 = false) {
  const int groups_per_token = k * f / 16;
  const int NG = T * groups_per_token;
  if (wide6 && groups_per_token % 6 == 0 && NG / 6 >= 2 * ncu) return 6;
  int best = 1;
  int64_t best_cost = -1;
  for (int g = 3; g >= 1; g--) {
    if (groups_per_token % g) continue;
    const int64_t blocks = NG / g;
    const int64_t cost = ((blocks + ncu - 1) / ncu) * g;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = g;
    }
  }
  return best;
}

// CUs of the current device (cached per device by launch_shape)
hipError_t cu_count(int* n) {
  int per_cu = 0;
  return launch_shape(nullptr, 0, 0, 0, &per_cu, n);
}

}  // namespace

size_t decode_quant_bytes(int T, int k, int d, int f) { return ws_layout(T, k, d, f).total; }

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t s) {
  if (L.T == 0) return hipSuccess;
  DecodeArgs a{};
  a.gate = make_qmat(L.w_gate, L.fmt_gate_up, L.E, L.f, L.d);
  a.up = make_qmat(L.w_up, L.fmt_gate_up, L.E, L.f, L.d);
  a.down = make_qmat(L.w_down, L.fmt_down, L.E, L.d, L.f);
  const int fs = L.has_shared ? L.fmt_shared : FMT_Q8;
  if (L.has_shared) {
    a.s_gate = make_qmat(L.s_gate, fs, 1, L.f, L.d);
    a.s_up = make_qmat(L.s_up, fs, 1, L.f, L.d);
    a.s_down = make_qmat(L.s_down, fs, 1, L.d, L.f);
  } else {
    a.s_gate = a.s_up = a.s_down = a.gate;
  }
  a.grid = L.grid;
  a.vq_cb = L.vq_cb;
  a.w_router = L.w_router;
  a.E = L.E;
  a.d = L.d;
  a.f = L.f;
  a.k = L.k;
  a.T = L.T;
  a.has_shared = L.has_shared;
  a.fused_topk = L.fused_topk;
  a.x = L.x;
  a.x_dtype = L.x_dtype;
  a.z = L.z;
  a.idx = L.idx;
  a.wt = L.wt;
  a.idx_out = L.idx_out;
  a.wt_out = L.wt_out;
  a.router_bias = L.router_bias;
  a.zkey = L.zkey;
  a.down_gain = L.down_gain;
  const DecodeWsLayout W = ws_layout(L.T, L.k, L.d, L.f);
  uint8_t* q = static_cast<uint8_t*>(L.quant);
  a.xq = q + W.xq;
  a.xs = reinterpret_cast<float*>(q + W.xs);
  a.xq_s = q + W.xq_s;
  a.xs_s = reinterpret_cast<float*>(q + W.xs_s);
  a.shared_k2 = L.has_shared && L.T == 1;
  // several tokens with routing in the first launch: that launch quantizes x
  // for the shared gate/up too, which the planning launch's blocks copy
  a.xs_global = L.has_shared && L.T >= 2 && !is_vq(L.fmt_gate_up) && L.fused_topk;
  a.hsh = reinterpret_cast<float*>(q + W.hsh);
  a.hq = q + W.hq;
  a.hs = reinterpret_cast<float*>(q + W.hs);
  a.hf = reinterpret_cast<float*>(q + W.hf);
  a.plan = reinterpret_cast<int*>(q + W.plan);
  a.umax = L.E < L.T * L.k ? L.E : L.T * L.k;
  a.y = L.y;
  int ncu = 256;
  if (hipError_t e = cu_count(&ncu); e != hipSuccess) return e;

  // Several tokens (block formats) take the planning launch, which also runs
  // their shared gate/up (plan_shared_kernel); otherwise the first launch
  // does (more than one token) or the second (one token).
  const bool plan_path = L.T >= 2 && !is_vq(L.fmt_gate_up);
  const int pw_s = fs == FMT_Q8 ? 16 : 64;
  const int rps_s = L.d / pw_s >= 64 ? 1 : 64 / (L.d / pw_s);
  const int64_t sb = 2 * rps_s * row_bytes(fs, L.d);  // bytes of one shared gate/up step
  // launch 1: router blocks of epb experts, shared blocks of spb steps, all
  // streaming about the same bytes
  K1Plan pl{};
  {
    const int n_router = L.fused_topk ? L.E : 0;
    pl.n_steps = L.has_shared && !a.shared_k2 && !plan_path ? L.f / rps_s : 0;
    const int64_t rb = (int64_t)L.d * 4;
    const int64_t total = n_router * rb + (int64_t)pl.n_steps * sb;
    int64_t nb = total / (32 << 10);
    nb = nb < 1 ? 1 : (nb > ncu ? ncu : nb);
    const double per_block = (double)total / (double)nb;
    pl.epb = (int)(per_block / (double)rb + 0.5);
    pl.epb = pl.epb < 1 ? 1 : (pl.epb > WAVES - 1 ? WAVES - 1 : pl.epb);  // the last wave quantizes x
    pl.n_rb = (n_router + pl.epb - 1) / pl.epb;
    if (pl.n_steps > 0) {
      int64_t n_sb = nb - pl.n_rb;
      if (n_sb < 1) n_sb = 1;
      pl.spb = (int)((pl.n_steps + n_sb - 1) / n_sb);
      pl.n_sb = (pl.n_steps + pl.spb - 1) / pl.spb;
    } else {
      pl.spb = 1;
      pl.n_sb = 0;
    }
    // x for the routed gate/up: by the router blocks' last waves, or without a
    // router by blocks of its own, one octet of chunks per wave
    const int n_oct = (L.T * (L.d / 64) + 7) / 8;
    pl.n_xb = pl.n_rb == 0 ? (n_oct + WAVES - 1) / WAVES : 0;
  }
  // (several tokens with the caller's routes: the planning launch also
  // quantizes x, and there is no first launch)
  const bool merged = plan_path && !L.fused_topk;
  if (!merged) {
    const int pid = prof_begin("decode_router", s);
    hipError_t e = launch_k1(a, pl, fs, nib_layout(L.fmt_gate_up), s);
    prof_end(pid, s);
    if (e != hipSuccess) return e;
  }

  // Several tokens (block formats): the top-k and the distinct experts in a
  // small launch of their own, then gate/up and down over the distinct
  // experts, each expert's codes loaded once for all its routes.
  if (plan_path) {
    {
      hipError_t e;
      const int pid = prof_begin("decode_plan", s);
      if (L.has_shared || merged) {
        // block 0 the plan; then the shared gate/up blocks, about 32 KB of
        // weights each; then (merged) the x blocks
        K1Plan ps{};
        ps.n_rb = 1;
        if (L.has_shared) {
          ps.n_steps = L.f / rps_s;
          int64_t nb = (int64_t)ps.n_steps * sb / (32 << 10);
          nb = nb < 1 ? 1 : (nb > ncu ? ncu : nb);
          ps.spb = (int)((ps.n_steps + nb - 1) / nb);
          ps.n_sb = (ps.n_steps + ps.spb - 1) / ps.spb;
        }
        ps.n_xb = merged ? pl.n_xb : 0;
        e = launch_plan_shared(a, ps, fs, nib_layout(L.fmt_gate_up), s);
      } else {
        e = launch_plan(a, s);
      }
      prof_end(pid, s);
      if (e != hipSuccess) return e;
    }
    {  // per token, the routes from the plan
      DecodeArgs b = a;
      b.fused_topk = 0;
      const int pid = prof_begin("decode_gateup", s);
      const int g = gcnt_of(L.k, L.f, L.T, ncu, true);
      hipError_t e = launch_k2(b, L.fmt_gate_up, fs, g, L.T * L.k * L.f / 16 / g, nib_layout(L.fmt_down), s);
      prof_end(pid, s);
      if (e != hipSuccess) return e;
    }
    // (rows of more than 2048 inputs: the one-token kernel, per token)
    const int pid = prof_begin("decode_down_combine", s);
    hipError_t e = L.f <= 2048 ? launch_k3u(a, L.fmt_down, fs, s) : launch_k3(a, L.fmt_down, fs, s);
    prof_end(pid, s);
    return e;
  }

  // launch 2: groups of 16 routed h rows, GCNT per block, blocks never
  // straddling a token
  {
    const int best = gcnt_of(L.k, L.f, L.T, ncu);
    const int NG = L.T * L.k * L.f / 16;
    const int pid = prof_begin("decode_gateup", s);
    hipError_t e = launch_k2(a, L.fmt_gate_up, fs, best, NG / best, nib_layout(L.fmt_down), s);
    prof_end(pid, s);
    if (e != hipSuccess) return e;
  }
  {
    const int pid = prof_begin("decode_down_combine", s);
    hipError_t e = launch_k3(a, L.fmt_down, fs, s);
    prof_end(pid, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qmoe
