// C ABI of the chunkwise mLSTM forward pass: argument validation, workspace
// layout and launch of the two stages.  See include/mlstm_tfla.h for the
// contract of every entry point.
#include <math.h>
#include <initializer_list>
#include <mutex>
#include <stdint.h>

#include "kernels.h"
#include "mlstm_tfla.h"

namespace {

using mlstm::GatesParams;
using mlstm::HintraParams;
using mlstm::StatesParams;

constexpr int kMaxChunk = 1024;
constexpr int kMinChunk = 16;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool fused_supported(const mlstm_fw_desc_t* d) {
  return d->precision == MLSTM_PREC_SPLIT &&
         mlstm::walk_supported(d->DHQK, d->DHV, d->chunk_size, d->qkv_dtype == MLSTM_BF16, true);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool packed_layout(const mlstm_fw_desc_t* d);

// The blocked schedule runs the wide kernels with the row-tile states kernel
// (one workgroup per head and row tile of the state, all value columns).
bool blocked_supported(const mlstm_fw_desc_t* d) {
  return d->precision != MLSTM_PREC_F64 && packed_layout(d) && mlstm::rows_tile_rows(d->DHQK, d->DHV) > 0;
}

// int16-coded chunk states: written by the row-tile states kernel in one
// segment and read by the wide intra-chunk kernel, so the wide family with
// split operands and a row-tile shape, on the two-stage schedule (the fused
// walker hands no states over; the blocked schedule keeps the pair form).
bool codes_supported(const mlstm_fw_desc_t* d) {
  return d->precision == MLSTM_PREC_SPLIT && packed_layout(d) && mlstm::rows_tile_rows(d->DHQK, d->DHV) > 0 &&
         d->schedule != MLSTM_SCHED_FUSED && d->schedule != MLSTM_SCHED_BLOCKED;
}

// Chunk states of one block of the blocked schedule, over all heads: half the
// 256 MB Infinity Cache, so that a block's states, written by the states
// kernel, are still there when the intra-chunk kernel reads them.
constexpr size_t kBlockStateBytes = size_t(128) << 20;

// Chunks per block of the blocked schedule (at least one).
int block_chunks(const mlstm_fw_desc_t* d) {
  const int Nc = (d->S + d->chunk_size - 1) / d->chunk_size;
  const size_t per_chunk = (size_t)d->B * d->NH * d->DHQK * d->DHV * sizeof(float);
  size_t k = d->block_chunks > 0 ? (size_t)d->block_chunks : kBlockStateBytes / per_chunk;
  if (k < 1) k = 1;
  if (k > (size_t)(Nc > 1 ? Nc : 1)) k = Nc > 1 ? Nc : 1;
  return (int)k;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int validate_desc(const mlstm_fw_desc_t* d) {
  if (!d) return MLSTM_E_NULLPTR;
  if (d->reserved != 0) return MLSTM_E_ARG;
  if (d->state_codes != MLSTM_STATES_SPLIT && d->state_codes != MLSTM_STATES_I16) return MLSTM_E_ARG;
  if (d->block_chunks < 0) return MLSTM_E_ARG;
  if (d->schedule != MLSTM_SCHED_AUTO && d->schedule != MLSTM_SCHED_TWO_STAGE && d->schedule != MLSTM_SCHED_FUSED &&
      d->schedule != MLSTM_SCHED_BLOCKED)
    return MLSTM_E_ARG;
  if (d->qkv_dtype != MLSTM_F32 && d->qkv_dtype != MLSTM_BF16) return MLSTM_E_DTYPE;
  if (d->h_dtype != MLSTM_F32 && d->h_dtype != MLSTM_BF16) return MLSTM_E_DTYPE;
  if (d->gate != MLSTM_GATE_EXP && d->gate != MLSTM_GATE_SIG) return MLSTM_E_ARG;
  if (d->precision != MLSTM_PREC_SPLIT && d->precision != MLSTM_PREC_F16 && d->precision != MLSTM_PREC_F64)
    return MLSTM_E_ARG;
  if (!isfinite(d->qk_scale) || !isfinite(d->eps) || d->eps < 0.0f) return MLSTM_E_ARG;
  if (d->B < 1 || d->NH < 1 || d->S < 0) return MLSTM_E_SHAPE;
  const bool dk_ok = d->DHQK == 64 || d->DHQK == 128 || d->DHQK == 256 || d->DHQK == 512;
  if (!dk_ok) return MLSTM_E_SHAPE;
  if (d->DHV < 64 || d->DHV > 512 || d->DHV % 64 != 0) return MLSTM_E_SHAPE;
  if (d->qkv_dtype == MLSTM_F32 && d->DHQK > 256) return MLSTM_E_UNSUPPORTED;
  if (!is_pow2(d->chunk_size) || d->chunk_size < kMinChunk || d->chunk_size > kMaxChunk) return MLSTM_E_CHUNK;
  if (d->tile_lq != 0 && d->tile_lq != 64 && d->tile_lq != 128) return MLSTM_E_CHUNK;
  if (d->tile_lkv != 0 && d->tile_lkv != 64 && d->tile_lkv != 128) return MLSTM_E_CHUNK;
  if (d->tile_lq > d->chunk_size || d->tile_lkv > d->chunk_size) return MLSTM_E_CHUNK;
  // 128-key tiles hold 128 full key rows in LDS: DHQK <= 256 (<= 128 for float32).
  if (d->tile_lkv == 128 && d->DHQK > (d->qkv_dtype == MLSTM_F32 ? 128 : 256)) return MLSTM_E_UNSUPPORTED;
  // Grid and index limits.
  const int64_t BH = (int64_t)d->B * d->NH;
  const int64_t Nc = ((int64_t)d->S + d->chunk_size - 1) / d->chunk_size;
  if (BH > (1 << 30)) return MLSTM_E_SHAPE;
  if (BH * Nc * (d->chunk_size > 64 ? d->chunk_size / 64 : 1) > 0x7fffffffLL) return MLSTM_E_SHAPE;  // grid.x bound
  // Per-head byte extents and row offsets of the buffer-resource kernels are
  // 32-bit: a head's largest float32 row block stays below 2 GiB.
  if ((int64_t)d->S * (int64_t)(d->DHQK > d->DHV ? d->DHQK : d->DHV) >= (1LL << 29)) return MLSTM_E_SHAPE;
  if (d->schedule == MLSTM_SCHED_FUSED && !fused_supported(d)) return MLSTM_E_UNSUPPORTED;
  if (d->schedule == MLSTM_SCHED_BLOCKED && !blocked_supported(d)) return MLSTM_E_UNSUPPORTED;
  if (d->state_codes == MLSTM_STATES_I16 && !codes_supported(d)) return MLSTM_E_UNSUPPORTED;
  return MLSTM_OK;
}

// Whether mlstm_chunkwise_fw runs the fused walker for a valid descriptor.
// The automatic schedule takes it wherever it covers the shape and no tile
// sizes of the two-stage kernels were asked for: on the 7B-shaped workloads
// it is the faster path for both gates.
bool use_fused(const mlstm_fw_desc_t* d) {
  if (d->schedule == MLSTM_SCHED_FUSED) return true;
  return d->schedule == MLSTM_SCHED_AUTO && d->tile_lq == 0 && d->tile_lkv == 0 && fused_supported(d);
}

struct WsLayout {
  size_t c_off, n_off, m_off, g_off, ml_off, cy_off, cs_off, total;
};

// Per-position gate terms: read by both wide-tile stages (the walker forms
// its own).
bool needs_gates(const mlstm_fw_desc_t* d) { return packed_layout(d) && d->schedule != MLSTM_SCHED_FUSED; }

WsLayout ws_layout(const mlstm_fw_desc_t* d) {
  const size_t BH = (size_t)d->B * d->NH;
  const bool blocked = d->schedule == MLSTM_SCHED_BLOCKED;
  // chunk-state slots per head: every chunk boundary, or one block's
  const size_t Nc1 = blocked ? (size_t)block_chunks(d) + 1
                             : (size_t)((d->S + d->chunk_size - 1) / d->chunk_size) + 1;
  const size_t el = d->precision == MLSTM_PREC_F64 ? sizeof(double) : sizeof(float);
  const bool states = d->schedule != MLSTM_SCHED_FUSED;  // chunk states can be formed
  const bool codes = d->state_codes == MLSTM_STATES_I16;
  WsLayout w;
  w.c_off = 0;
  size_t off = states ? round_up(BH * Nc1 * d->DHQK * d->DHV * (codes ? sizeof(int16_t) : el), 256) : 0;
  w.n_off = off;
  if (states && d->gate == MLSTM_GATE_EXP) off += round_up(BH * Nc1 * d->DHQK * el, 256);
  w.m_off = off;
  if (states && d->gate == MLSTM_GATE_EXP) off += round_up(BH * Nc1 * el, 256);
  w.g_off = off;
  if (needs_gates(d)) off += round_up(BH * (size_t)d->S * sizeof(float) * (d->gate == MLSTM_GATE_EXP ? 3 : 2), 256);
  // stabilisers of segment-local runs of the states kernel
  w.ml_off = off;
  if (states && !blocked && packed_layout(d)) off += round_up(BH * Nc1 * sizeof(float), 256);
  // blocked schedule: the state handed from one block to the next, twice
  // (read by one block while the next is written): C, n, m as float32
  w.cy_off = off;
  if (blocked)
    off += 2 * (round_up(BH * d->DHQK * d->DHV * sizeof(float), 256) + round_up(BH * d->DHQK * sizeof(float), 256) +
                round_up(BH * sizeof(float), 256));
  // int16-coded states: one float32 scale per 16 x 32 fragment
  w.cs_off = off;
  if (states && codes) off += round_up(BH * Nc1 * (d->DHQK / 16) * (d->DHV / 32) * sizeof(float), 256);
  w.total = off;
  return w;
}

int check_sig_nulls(const mlstm_fw_desc_t* d, const void* a, const void* b, const void* c, const void* e) {
  if (d->gate == MLSTM_GATE_SIG && (a || b || c || e)) return MLSTM_E_UNSUPPORTED;
  return MLSTM_OK;
}

int check_f32_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return MLSTM_E_ALIGN;
  return MLSTM_OK;
}

float resolve_scale(const mlstm_fw_desc_t* d) {
  return d->qk_scale > 0.0f ? d->qk_scale : 1.0f / sqrtf((float)d->DHQK);
}

// The wide kernels (bf16 inputs, large head dims) keep the chunk states in
// the packed fragment layout; every other shape uses float32 row-major
// states.  Both layouts take the same number of bytes.
bool packed_layout(const mlstm_fw_desc_t* d) {
  if (d->precision == MLSTM_PREC_F64) return false;
  const int tq = d->tile_lq ? d->tile_lq : 64;
  return mlstm::hintra_wide_supported(d->DHQK, d->DHV, d->chunk_size, tq, d->qkv_dtype == MLSTM_BF16);
}

struct WsPtrs {
  float* C;
  float* n;
  float* m;
  float* gb2;  // gate terms (wide-tile path), else null
  float* gu2;
  float* gpm2;
  float* m_local;  // segment-local stabilisers (wide-tile path), else null
  float* cy_C[2];  // blocked schedule: the state between blocks, else null
  float* cy_n[2];
  float* cy_m[2];
  float* C_scales;  // int16-coded states: fragment scales, else null (C then holds the codes)
};

WsPtrs ws_ptrs(const mlstm_fw_desc_t* d, void* workspace) {
  const WsLayout w = ws_layout(d);
  char* ws = static_cast<char*>(workspace);
  WsPtrs r;
  r.C = reinterpret_cast<float*>(ws + w.c_off);
  r.n = d->gate == MLSTM_GATE_EXP ? reinterpret_cast<float*>(ws + w.n_off) : nullptr;
  r.m = d->gate == MLSTM_GATE_EXP ? reinterpret_cast<float*>(ws + w.m_off) : nullptr;
  r.gb2 = r.gu2 = r.gpm2 = r.m_local = nullptr;
  r.C_scales = d->state_codes == MLSTM_STATES_I16 && d->schedule != MLSTM_SCHED_FUSED
                   ? reinterpret_cast<float*>(ws + w.cs_off)
                   : nullptr;
  const bool blocked = d->schedule == MLSTM_SCHED_BLOCKED;
  if (packed_layout(d) && d->schedule != MLSTM_SCHED_FUSED && !blocked)
    r.m_local = reinterpret_cast<float*>(ws + w.ml_off);
  for (int i = 0; i < 2; ++i) r.cy_C[i] = r.cy_n[i] = r.cy_m[i] = nullptr;
  if (blocked) {
    const size_t BH = (size_t)d->B * d->NH;
    const size_t cb = round_up(BH * d->DHQK * d->DHV * sizeof(float), 256);
    const size_t nb = round_up(BH * d->DHQK * sizeof(float), 256), mb = round_up(BH * sizeof(float), 256);
    char* c = ws + w.cy_off;
    for (int i = 0; i < 2; ++i) {
      r.cy_C[i] = reinterpret_cast<float*>(c);
      r.cy_n[i] = reinterpret_cast<float*>(c + cb);
      r.cy_m[i] = reinterpret_cast<float*>(c + cb + nb);
      c += cb + nb + mb;
    }
  }
  if (needs_gates(d)) {
    const size_t n = (size_t)d->B * d->NH * d->S;
    r.gb2 = reinterpret_cast<float*>(ws + w.g_off);
    r.gu2 = r.gb2 + n;
    r.gpm2 = d->gate == MLSTM_GATE_EXP ? r.gu2 + n : nullptr;
  }
  return r;
}

int check_workspace(const mlstm_fw_desc_t* d, const void* workspace, size_t workspace_bytes) {
  const WsLayout w = ws_layout(d);
  if (w.total > 0 && (!workspace || workspace_bytes < w.total)) return MLSTM_E_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return MLSTM_E_WORKSPACE;
  return MLSTM_OK;
}

hipError_t run_gates(const mlstm_fw_desc_t* d, const float* i_pre, const float* f_pre, const WsPtrs& ws,
                     hipStream_t stream) {
  GatesParams g;
  g.i_pre = i_pre;
  g.f_pre = f_pre;
  g.gb2 = ws.gb2;
  g.gu2 = ws.gu2;
  g.gpm2 = ws.gpm2;
  g.BH = d->B * d->NH;
  g.S = d->S;
  g.L = d->chunk_size;
  g.Nc = (d->S + d->chunk_size - 1) / d->chunk_size;
  return mlstm::launch_gates(g, d->gate == MLSTM_GATE_SIG, stream);
}

int run_fused(const mlstm_fw_desc_t* d, const void* Q, const void* K, const void* V, const float* i_pre,
              const float* f_pre, const float* C0, const float* n0, const float* m0, const WsPtrs& ws, void* H,
              float* C_out, float* n_out, float* m_out, float* m_rows, float* den_rows, hipStream_t stream) {
  (void)ws;
  mlstm::WalkParams p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.C0 = C0;
  p.n0 = n0;
  p.m0 = m0;
  p.H = H;
  p.C_out = C_out;
  p.n_out = n_out;
  p.m_out = m_out;
  p.m_rows = m_rows;
  p.den_rows = den_rows;
  p.scale = resolve_scale(d);
  p.eps = d->eps;
  p.BH = d->B * d->NH;
  p.S = d->S;
  p.DK = d->DHQK;
  p.DV = d->DHV;
  p.L = d->chunk_size;
  p.Nc = (d->S + d->chunk_size - 1) / d->chunk_size;
  p.h_bf16 = d->h_dtype == MLSTM_BF16;
  const hipError_t e = mlstm::launch_walk(p, d->gate == MLSTM_GATE_SIG, stream);
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

// C_plain (packed layout only): also deliver the chunk states as float32
// row-major; plain_only: no intra-chunk kernel will read the packed copy.
int run_states(const mlstm_fw_desc_t* d, const void* K, const void* V, const float* i_pre, const float* f_pre,
               const float* C0, const float* n0, const float* m0, const WsPtrs& ws, float* C_out, float* n_out,
               float* m_out, hipStream_t stream, float* C_plain = nullptr, bool plain_only = false) {
  StatesParams p;
  p.K = K;
  p.V = V;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.C0 = C0;
  p.n0 = n0;
  p.m0 = m0;
  p.C_states = ws.C;
  p.n_states = ws.n;
  p.m_states = ws.m;
  p.C_out = C_out;
  p.n_out = n_out;
  p.m_out = m_out;
  p.gb2 = ws.gb2;
  p.gu2 = ws.gu2;
  p.gpm2 = ws.gpm2;
  p.m_local = ws.m_local;
  p.BH = d->B * d->NH;
  p.S = d->S;
  p.DK = d->DHQK;
  p.DV = d->DHV;
  p.L = d->chunk_size;
  p.Nc = (d->S + d->chunk_size - 1) / d->chunk_size;
  p.nseg = 1;
  p.cps = p.Nc;
  const bool bf16 = d->qkv_dtype == MLSTM_BF16;
  const bool sig = d->gate == MLSTM_GATE_SIG;
  const bool split = bf16 && d->precision == MLSTM_PREC_SPLIT;
  hipError_t e;
  if (d->precision == MLSTM_PREC_F64) e = mlstm::launch_states_f64(p, bf16, sig, stream);
  else if (packed_layout(d)) {
    p.C_plain = C_plain;
    p.plain_only = C_plain && plain_only;
    p.C_scales = ws.C_scales;
    e = run_gates(d, i_pre, f_pre, ws, stream);
    if (e == hipSuccess) e = mlstm::launch_states_wide(p, sig, split, stream);
  }
  else e = mlstm::launch_states(p, bf16, sig, split, stream);
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

int run_hintra(const mlstm_fw_desc_t* d, const void* Q, const void* K, const void* V, const float* i_pre,
               const float* f_pre, const WsPtrs& ws, void* H, float* m_rows, float* den_rows,
               hipStream_t stream, const void* dH = nullptr, bool dh_bf16 = false, float* ginvz = nullptr,
               float* gdelta = nullptr) {
  if (d->S == 0) return MLSTM_OK;
  HintraParams p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.C_states = ws.C;
  p.n_states = ws.n;
  p.m_states = ws.m;
  p.H = H;
  p.m_rows = m_rows;
  p.den_rows = den_rows;
  p.gb2 = ws.gb2;
  p.gu2 = ws.gu2;
  p.gpm2 = ws.gpm2;
  p.scale = resolve_scale(d);
  p.eps = d->eps;
  p.BH = d->B * d->NH;
  p.S = d->S;
  p.DK = d->DHQK;
  p.DV = d->DHV;
  p.L = d->chunk_size;
  p.Nc = (d->S + d->chunk_size - 1) / d->chunk_size;
  p.h_bf16 = d->h_dtype == MLSTM_BF16;
  p.tile_lq = d->tile_lq ? d->tile_lq : 64;
  p.tile_lkv = d->tile_lkv ? d->tile_lkv : 64;
  // backward recompute: the row terms of the gradient instead of H (wide
  // kernel; dH is float32 or bf16 as h_dtype of the caller's descriptor says)
  p.dH = dH;
  p.dh_bf16 = dh_bf16;
  p.ginvz = ginvz;
  p.gdelta = gdelta;
  p.C_scales = ws.C_scales;
  const bool bf16 = d->qkv_dtype == MLSTM_BF16;
  const bool sig = d->gate == MLSTM_GATE_SIG;
  const bool split = bf16 && d->precision == MLSTM_PREC_SPLIT;
  hipError_t e;
  if (d->precision == MLSTM_PREC_F64) e = mlstm::launch_hintra_f64(p, bf16, sig, stream);
  else if (packed_layout(d)) e = mlstm::launch_hintra_wide(p, sig, split, stream);
  else e = mlstm::launch_hintra(p, bf16, sig, split, stream);
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

// Blocked schedule: the two stages per block of chunks, over all heads.  The
// states kernel starts each block from the state the previous block ended
// in (the initial state for the first) and writes the block's chunk states
// with plain stores; the intra-chunk kernel reads them back while they are
// still in the Infinity Cache.  The last block ends in the final state.
int run_blocked(const mlstm_fw_desc_t* d, const void* Q, const void* K, const void* V, const float* i_pre,
                const float* f_pre, const float* C0, const float* n0, const float* m0, const WsPtrs& ws, void* H,
                float* C_out, float* n_out, float* m_out, float* m_rows, float* den_rows, hipStream_t stream) {
  const int Nc = (d->S + d->chunk_size - 1) / d->chunk_size;
  const int k = block_chunks(d);
  const bool sig = d->gate == MLSTM_GATE_SIG;
  const bool split = d->precision == MLSTM_PREC_SPLIT;
  hipError_t e = hipSuccess;
  if (d->S > 0) e = run_gates(d, i_pre, f_pre, ws, stream);
  const int nblk = Nc > 0 ? (Nc + k - 1) / k : 1;
  for (int b = 0; b < nblk && e == hipSuccess; ++b) {
    const int c_lo = b * k, c_hi = Nc < c_lo + k ? Nc : c_lo + k;
    const bool last = b + 1 == nblk;
    StatesParams p;
    p.K = K;
    p.V = V;
    p.i_pre = i_pre;
    p.f_pre = f_pre;
    p.C0 = b == 0 ? C0 : ws.cy_C[b & 1];
    p.n0 = b == 0 ? n0 : ws.cy_n[b & 1];
    p.m0 = b == 0 ? m0 : ws.cy_m[b & 1];
    p.C_states = ws.C;
    p.n_states = ws.n;
    p.m_states = ws.m;
    p.C_out = last ? C_out : ws.cy_C[(b + 1) & 1];
    p.n_out = last ? n_out : (sig ? nullptr : ws.cy_n[(b + 1) & 1]);
    p.m_out = last ? m_out : (sig ? nullptr : ws.cy_m[(b + 1) & 1]);
    p.gb2 = ws.gb2;
    p.gu2 = ws.gu2;
    p.gpm2 = ws.gpm2;
    p.m_local = nullptr;
    p.BH = d->B * d->NH;
    p.S = d->S;
    p.DK = d->DHQK;
    p.DV = d->DHV;
    p.L = d->chunk_size;
    p.Nc = Nc;
    p.c_lo = c_lo;
    p.c_hi = c_hi;
    p.slots = k + 1;
    p.nt_states = 0;
    e = mlstm::launch_states_rows_range(p, sig, split, stream);
    if (e != hipSuccess || d->S == 0) break;
    HintraParams h;
    h.Q = Q;
    h.K = K;
    h.V = V;
    h.i_pre = i_pre;
    h.f_pre = f_pre;
    h.C_states = ws.C;
    h.n_states = ws.n;
    h.m_states = ws.m;
    h.H = H;
    h.m_rows = m_rows;
    h.den_rows = den_rows;
    h.gb2 = ws.gb2;
    h.gu2 = ws.gu2;
    h.gpm2 = ws.gpm2;
    h.scale = resolve_scale(d);
    h.eps = d->eps;
    h.BH = d->B * d->NH;
    h.S = d->S;
    h.DK = d->DHQK;
    h.DV = d->DHV;
    h.L = d->chunk_size;
    h.Nc = Nc;
    h.h_bf16 = d->h_dtype == MLSTM_BF16;
    h.tile_lq = d->tile_lq ? d->tile_lq : 64;
    h.tile_lkv = d->tile_lkv ? d->tile_lkv : 64;
    h.c_lo = c_lo;
    h.c_hi = c_hi;
    h.slots = k + 1;
    e = mlstm::launch_hintra_wide(h, sig, split, stream);
  }
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

// The chunk states of a two-stage workspace as float32 row-major arrays.
int unpack_states(const mlstm_fw_desc_t* d, const WsPtrs& ws, float* C_states, float* n_states, float* m_states,
                  hipStream_t s) {
  const long long n = (long long)d->B * d->NH * ((d->S + d->chunk_size - 1) / d->chunk_size + 1);
  hipError_t e = hipSuccess;
  if (d->precision == MLSTM_PREC_F64) {
    if (C_states) e = mlstm::launch_narrow_f64(ws.C, C_states, n * d->DHQK * d->DHV, s);
    if (e == hipSuccess && n_states) e = mlstm::launch_narrow_f64(ws.n, n_states, n * d->DHQK, s);
    if (e == hipSuccess && m_states) e = mlstm::launch_narrow_f64(ws.m, m_states, n, s);
    return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
  }
  if (C_states) {
    if (packed_layout(d)) {
      e = mlstm::launch_unpack_states(ws.C, C_states, n, d->DHQK, d->DHV, s, ws.C_scales);
    } else {
      e = hipMemcpyAsync(C_states, ws.C, (size_t)n * d->DHQK * d->DHV * sizeof(float), hipMemcpyDeviceToDevice, s);
    }
  }
  if (e == hipSuccess && n_states)
    e = hipMemcpyAsync(n_states, ws.n, (size_t)n * d->DHQK * sizeof(float), hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && m_states)
    e = hipMemcpyAsync(m_states, ws.m, (size_t)n * sizeof(float), hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

// ---- backward pass
// The backward recomputes the forward quantities it needs with the two-stage
// kernels (the walker forms no chunk states and no per-row normaliser), with
// H in float32.
// The gradient does not depend on how the sequence is cut into chunks, so
// the backward picks its own: chunks below 64 rows run as chunks of 64 (the
// gradient kernels work in 64-row tiles), longer ones as chunks of at most
// 256 rows, or 128 when the heads alone give the row-tile state-gradient
// kernel a workgroup per CU (BH * DHQK / 64 >= 256 CUs).  The intra-chunk
// gradient tiles grow with the chunk length, the sequential state-gradient
// recurrence with the number of chunks: at 65536 tokens and 8 heads chunks of
// 256 take 13.0 ms (16.9 at 1024, 13.8 at 128); at 8192 tokens and 64 heads
// chunks of 128 take 6.9 ms (7.4 at 256, 7.8 at 64).
int bw_max_chunk(const mlstm_fw_desc_t* d) {
  return (int64_t)d->B * d->NH * (d->DHQK / 64) >= 256 ? 128 : 256;
}

mlstm_fw_desc_t bw_fw_desc(const mlstm_fw_desc_t* d) {
  mlstm_fw_desc_t r = *d;
  r.state_codes = MLSTM_STATES_SPLIT;  // the recompute keeps its states as hi + lo pairs
  r.schedule = MLSTM_SCHED_TWO_STAGE;
  r.h_dtype = MLSTM_F32;
  if (r.chunk_size < 64) r.chunk_size = 64;
  if (r.chunk_size > bw_max_chunk(d)) r.chunk_size = bw_max_chunk(d);
  // the library's own tiles (64-row intra-chunk tiles hold whole rows, which
  // the row terms of the gradient need); the result does not depend on them
  r.tile_lq = r.tile_lkv = 0;
  return r;
}

// Exp gate on the wide kernels: the recompute forms the row terms of the
// gradient (1/z and delta) in the intra-chunk kernel's epilogue from dH, and
// H is never stored; elsewhere it stores H for the gradient stage.
bool bw_delta_in_recompute(const mlstm_fw_desc_t* d2) {
  return d2->gate == MLSTM_GATE_EXP && packed_layout(d2);
}

struct BwLayout {
  size_t Cst, nst, mst, H, mrows, den, gb, gsrc, ginvz, gdelta, dC, dn, qdq, kdk, gtot, dC0, dn0, dS, seg, segn, total;
  int nseg, cps;  // sequence segments of the state-gradient recurrence
};

// Forward workspace first, then the backward's own regions, each 256-byte aligned.
BwLayout bw_layout(const mlstm_fw_desc_t* d2) {
  const size_t BH = (size_t)d2->B * d2->NH, S = (size_t)d2->S, DK = d2->DHQK, DV = d2->DHV;
  const size_t Nc = (S + d2->chunk_size - 1) / d2->chunk_size;
  const bool ex = d2->gate == MLSTM_GATE_EXP;
  const size_t f = sizeof(float);
  BwLayout l;
  size_t off = round_up(ws_layout(d2).total, 256);
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes, 256);
    return at;
  };
  l.Cst = take(BH * (Nc + 1) * DK * DV * f);
  l.nst = take(ex ? BH * (Nc + 1) * DK * f : 0);
  l.mst = take(ex ? BH * (Nc + 1) * f : 0);
  l.H = take(ex && !bw_delta_in_recompute(d2) ? BH * S * DV * f : 0);
  l.mrows = take(ex ? BH * S * f : 0);
  l.den = take(ex ? BH * S * f : 0);
  l.gb = take(BH * S * f);
  l.gsrc = take(BH * S * f);
  l.ginvz = take(ex ? BH * S * f : 0);
  l.gdelta = take(ex ? BH * S * f : 0);
  l.dC = take(BH * Nc * DK * DV * f);
  l.dn = take(ex ? BH * Nc * DK * f : 0);
  l.qdq = take(BH * S * f);
  l.kdk = take(BH * S * f);
  l.gtot = take(BH * ((S + 1023) / 1024 + 32) * f);
  l.dC0 = take(BH * DK * DV * f);
  l.dn0 = take(ex ? BH * DK * f : 0);
  const size_t nT = (size_t)d2->chunk_size / 64;
  l.dS = take(d2->qkv_dtype == MLSTM_BF16 ? BH * Nc * (nT * (nT + 1) / 2) * 64 * 64 * f : 0);
  l.nseg = mlstm::bw_dstate_segments((int)BH, (int)DK, (int)DV, (int)Nc, d2->qkv_dtype == MLSTM_BF16, &l.cps);
  l.seg = take(l.nseg > 1 ? BH * l.nseg * DK * DV * f : 0);
  l.segn = take(l.nseg > 1 && ex ? BH * l.nseg * DK * f : 0);
  l.total = off;
  return l;
}

}  // namespace

extern "C" {

int mlstm_abi_version(void) { return MLSTM_ABI_VERSION; }

const char* mlstm_status_str(int status) {
  switch (status) {
    case MLSTM_OK: return "ok";
    case MLSTM_E_NULLPTR: return "null pointer";
    case MLSTM_E_SHAPE: return "unsupported shape";
    case MLSTM_E_CHUNK: return "unsupported chunk or tile size";
    case MLSTM_E_DTYPE: return "unknown dtype";
    case MLSTM_E_UNSUPPORTED: return "unsupported combination";
    case MLSTM_E_WORKSPACE: return "workspace missing or too small";
    case MLSTM_E_HIP: return "HIP launch failed";
    case MLSTM_E_ALIGN: return "misaligned pointer";
    case MLSTM_E_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

int mlstm_fw_validate(const mlstm_fw_desc_t* desc) { return validate_desc(desc); }

int64_t mlstm_fw_num_chunks(const mlstm_fw_desc_t* desc) {
  if (validate_desc(desc) != MLSTM_OK) return -1;
  return ((int64_t)desc->S + desc->chunk_size - 1) / desc->chunk_size;
}

int mlstm_fw_kernel_family(const mlstm_fw_desc_t* desc) {
  const int st = validate_desc(desc);
  if (st != MLSTM_OK) return -st;
  if (desc->precision == MLSTM_PREC_F64) return MLSTM_FAMILY_F64;
  if (use_fused(desc)) return MLSTM_FAMILY_FUSED;
  if (desc->schedule == MLSTM_SCHED_BLOCKED) return MLSTM_FAMILY_BLOCKED;
  return packed_layout(desc) ? MLSTM_FAMILY_WIDE : MLSTM_FAMILY_GENERIC;
}

size_t mlstm_fw_workspace_bytes(const mlstm_fw_desc_t* desc) {
  if (validate_desc(desc) != MLSTM_OK) return 0;
  return ws_layout(desc).total;
}

int mlstm_fw_states(const mlstm_fw_desc_t* desc, const void* K, const void* V, const float* i_pre,
                    const float* f_pre, const float* C0, const float* n0, const float* m0, void* workspace,
                    size_t workspace_bytes, float* C_out, float* n_out, float* m_out, void* stream) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->schedule == MLSTM_SCHED_FUSED || desc->schedule == MLSTM_SCHED_BLOCKED) return MLSTM_E_UNSUPPORTED;
  if (desc->S > 0 && (!K || !V || !i_pre || !f_pre)) return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n0, m0, n_out, m_out)) != MLSTM_OK) return st;
  if ((K && !aligned(K, 16)) || (V && !aligned(V, 16))) return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, C0, n0, m0, C_out, n_out, m_out})) != MLSTM_OK) return st;
  if ((st = check_workspace(desc, workspace, workspace_bytes)) != MLSTM_OK) return st;
  return run_states(desc, K, V, i_pre, f_pre, C0, n0, m0, ws_ptrs(desc, workspace), C_out, n_out, m_out,
                    static_cast<hipStream_t>(stream));
}

int mlstm_fw_hintra(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
                    const float* f_pre, const void* workspace, size_t workspace_bytes, void* H, float* m_rows,
                    float* den_rows, void* stream) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->schedule == MLSTM_SCHED_FUSED || desc->schedule == MLSTM_SCHED_BLOCKED) return MLSTM_E_UNSUPPORTED;
  if (desc->S > 0 && (!Q || !K || !V || !i_pre || !f_pre || !H)) return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, m_rows, den_rows, nullptr, nullptr)) != MLSTM_OK) return st;
  if ((Q && !aligned(Q, 16)) || (K && !aligned(K, 16)) || (V && !aligned(V, 16)) || (H && !aligned(H, 16)))
    return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, m_rows, den_rows})) != MLSTM_OK) return st;
  if ((st = check_workspace(desc, workspace, workspace_bytes)) != MLSTM_OK) return st;
  return run_hintra(desc, Q, K, V, i_pre, f_pre, ws_ptrs(desc, const_cast<void*>(workspace)), H, m_rows,
                    den_rows, static_cast<hipStream_t>(stream));
}

int mlstm_fw_unpack_states(const mlstm_fw_desc_t* desc, const void* workspace, size_t workspace_bytes,
                           float* C_states, float* n_states, float* m_states, void* stream) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->schedule == MLSTM_SCHED_FUSED || desc->schedule == MLSTM_SCHED_BLOCKED) return MLSTM_E_UNSUPPORTED;
  if ((st = check_sig_nulls(desc, n_states, m_states, nullptr, nullptr)) != MLSTM_OK) return st;
  if ((st = check_f32_ptrs({C_states, n_states, m_states})) != MLSTM_OK) return st;
  if ((st = check_workspace(desc, workspace, workspace_bytes)) != MLSTM_OK) return st;
  return unpack_states(desc, ws_ptrs(desc, const_cast<void*>(workspace)), C_states, n_states, m_states,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Host checks of the forward pass's arguments other than the workspace.
int check_fw_args(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
                  const float* f_pre, const float* C0, const float* n0, const float* m0, const void* H,
                  const float* C_out, const float* n_out, const float* m_out) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->S > 0 && (!Q || !K || !V || !i_pre || !f_pre || !H)) return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n0, m0, n_out, m_out)) != MLSTM_OK) return st;
  if ((Q && !aligned(Q, 16)) || (K && !aligned(K, 16)) || (V && !aligned(V, 16)) || (H && !aligned(H, 16)))
    return MLSTM_E_ALIGN;
  return check_f32_ptrs({i_pre, f_pre, C0, n0, m0, C_out, n_out, m_out});
}

// The forward pass on a checked workspace.
int run_fw(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
           const float* f_pre, const float* C0, const float* n0, const float* m0, void* H, float* C_out,
           float* n_out, float* m_out, float* m_rows, float* den_rows, void* workspace, hipStream_t s) {
  const WsPtrs ws = ws_ptrs(desc, workspace);
  if (use_fused(desc))
    return run_fused(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, ws, H, C_out, n_out, m_out, m_rows, den_rows, s);
  if (desc->schedule == MLSTM_SCHED_BLOCKED)
    return run_blocked(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, ws, H, C_out, n_out, m_out, m_rows, den_rows, s);
  const int st = run_states(desc, K, V, i_pre, f_pre, C0, n0, m0, ws, C_out, n_out, m_out, s);
  if (st != MLSTM_OK) return st;
  return run_hintra(desc, Q, K, V, i_pre, f_pre, ws, H, m_rows, den_rows, s);
}

// ---- workspace of the allocation-free forward pass: a static device array
// (each GPU that loads the library holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel: on the host it
// is only a stand-in, so its device address is looked up once per device
// with that device current, and that address is what the kernels get.
static __device__ __align__(256) unsigned char scratch[MLSTM_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch` per device, once looked up

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLSTM_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLSTM_E_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MLSTM_OK;
}

}  // namespace

extern "C" {

int mlstm_chunkwise_fw(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V,
                       const float* i_pre, const float* f_pre, const float* C0, const float* n0, const float* m0,
                       void* H, float* C_out, float* n_out, float* m_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = check_fw_args(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, H, C_out, n_out, m_out);
  if (st != MLSTM_OK) return st;
  if ((st = check_workspace(desc, workspace, workspace_bytes)) != MLSTM_OK) return st;
  return run_fw(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, H, C_out, n_out, m_out, nullptr, nullptr, workspace,
                static_cast<hipStream_t>(stream));
}

int mlstm_chunkwise_fw_rows(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V,
                            const float* i_pre, const float* f_pre, const float* C0, const float* n0,
                            const float* m0, void* H, float* C_out, float* n_out, float* m_out, float* m_rows,
                            float* den_rows, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_fw_args(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, H, C_out, n_out, m_out);
  if (st != MLSTM_OK) return st;
  if (desc->gate == MLSTM_GATE_SIG && (m_rows || den_rows)) return MLSTM_E_UNSUPPORTED;
  if ((st = check_f32_ptrs({m_rows, den_rows})) != MLSTM_OK) return st;
  if ((st = check_workspace(desc, workspace, workspace_bytes)) != MLSTM_OK) return st;
  return run_fw(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, H, C_out, n_out, m_out, m_rows, den_rows, workspace,
                static_cast<hipStream_t>(stream));
}

int mlstm_chunkwise_fw_noalloc(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V,
                               const float* i_pre, const float* f_pre, const float* C0, const float* n0,
                               const float* m0, void* H, float* C_out, float* n_out, float* m_out,
                               void* stream) {
  int st = check_fw_args(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, H, C_out, n_out, m_out);
  if (st != MLSTM_OK) return st;
  // the workspace of the kernels that run: where the automatic schedule
  // picks the fused walker, only its gate terms
  mlstm_fw_desc_t d = *desc;
  if (use_fused(&d)) d.schedule = MLSTM_SCHED_FUSED;
  const size_t need = ws_layout(&d).total;
  if (need > (size_t)MLSTM_NOALLOC_WORKSPACE_BYTES) return MLSTM_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_address(&ws)) != MLSTM_OK) return st;
  return run_fw(&d, Q, K, V, i_pre, f_pre, C0, n0, m0, H, C_out, n_out, m_out, nullptr, nullptr, ws,
                static_cast<hipStream_t>(stream));
}

int mlstm_recurrent_step(const mlstm_fw_desc_t* desc, const void* q, const void* k, const void* v,
                         const float* i_pre, const float* f_pre, const float* C_in, const float* n_in,
                         const float* m_in, void* h, float* C_out, float* n_out, float* m_out, void* stream) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->S != 1) return MLSTM_E_SHAPE;
  if (!q || !k || !v || !i_pre || !f_pre || !h || !C_out) return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n_in, m_in, n_out, m_out)) != MLSTM_OK) return st;
  // every workgroup of a head reads n_in / m_in while one of them writes the
  // new values: in-place update is allowed for C only
  if ((n_out && n_out == n_in) || (m_out && m_out == m_in)) return MLSTM_E_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(h, 16) || !aligned(C_out, 16) ||
      (C_in && !aligned(C_in, 16)))
    return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, n_in, m_in, n_out, m_out})) != MLSTM_OK) return st;
  mlstm::StepParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.C_in = C_in;
  p.n_in = n_in;
  p.m_in = m_in;
  p.h = h;
  p.C_out = C_out;
  p.n_out = n_out;
  p.m_out = m_out;
  p.scale = resolve_scale(desc);
  p.eps = desc->eps;
  p.BH = desc->B * desc->NH;
  p.DK = desc->DHQK;
  p.DV = desc->DHV;
  p.qkv_bf16 = desc->qkv_dtype == MLSTM_BF16;
  p.h_bf16 = desc->h_dtype == MLSTM_BF16;
  p.Cq_in = nullptr;
  p.Cs_in = nullptr;
  p.Cq_out = nullptr;
  p.Cs_out = nullptr;
  p.q8 = 0;
  const hipError_t e = mlstm::launch_step(p, desc->gate == MLSTM_GATE_SIG, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

int mlstm_recurrent_step_q8(const mlstm_fw_desc_t* desc, const void* q, const void* k, const void* v,
                            const float* i_pre, const float* f_pre, const int8_t* Cq_in, const float* Cs_in,
                            const float* n_in, const float* m_in, void* h, int8_t* Cq_out, float* Cs_out,
                            float* n_out, float* m_out, void* stream) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->S != 1) return MLSTM_E_SHAPE;
  if (!q || !k || !v || !i_pre || !f_pre || !h || !Cq_out || !Cs_out) return MLSTM_E_NULLPTR;
  if ((Cq_in == nullptr) != (Cs_in == nullptr)) return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n_in, m_in, n_out, m_out)) != MLSTM_OK) return st;
  if ((n_out && n_out == n_in) || (m_out && m_out == m_in)) return MLSTM_E_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(h, 16) || !aligned(Cq_out, 4) ||
      (Cq_in && !aligned(Cq_in, 4)) || !aligned(Cs_out, 16) || (Cs_in && !aligned(Cs_in, 16)))
    return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, n_in, m_in, n_out, m_out})) != MLSTM_OK) return st;
  mlstm::StepParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.C_in = nullptr;
  p.n_in = n_in;
  p.m_in = m_in;
  p.h = h;
  p.C_out = nullptr;
  p.n_out = n_out;
  p.m_out = m_out;
  p.Cq_in = Cq_in;
  p.Cs_in = Cs_in;
  p.Cq_out = Cq_out;
  p.Cs_out = Cs_out;
  p.q8 = 1;
  p.scale = resolve_scale(desc);
  p.eps = desc->eps;
  p.BH = desc->B * desc->NH;
  p.DK = desc->DHQK;
  p.DV = desc->DHV;
  p.qkv_bf16 = desc->qkv_dtype == MLSTM_BF16;
  p.h_bf16 = desc->h_dtype == MLSTM_BF16;
  const hipError_t e = mlstm::launch_step(p, desc->gate == MLSTM_GATE_SIG, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

int mlstm_state_q8_encode(const mlstm_fw_desc_t* desc, const float* C, int8_t* Cq, float* Cs, void* stream) {
  const int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (!C || !Cq || !Cs) return MLSTM_E_NULLPTR;
  if (!aligned(C, 4) || !aligned(Cs, 4)) return MLSTM_E_ALIGN;
  const hipError_t e = mlstm::launch_q8_encode(C, Cq, Cs, (long long)desc->B * desc->NH, desc->DHQK, desc->DHV,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

int mlstm_state_q8_decode(const mlstm_fw_desc_t* desc, const int8_t* Cq, const float* Cs, float* C, void* stream) {
  const int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (!C || !Cq || !Cs) return MLSTM_E_NULLPTR;
  if (!aligned(C, 4) || !aligned(Cs, 4)) return MLSTM_E_ALIGN;
  const hipError_t e = mlstm::launch_q8_decode(Cq, Cs, C, (long long)desc->B * desc->NH, desc->DHQK, desc->DHV,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

size_t mlstm_bw_workspace_bytes(const mlstm_fw_desc_t* desc) {
  if (validate_desc(desc) != MLSTM_OK) return 0;
  const mlstm_fw_desc_t d2 = bw_fw_desc(desc);
  return bw_layout(&d2).total;
}

// Where the recompute leaves the float32 chunk states: the backward's own
// region (written by the sig-gate wide states kernel, or narrowed from
// float64), or, for the generic kernels, their float32 workspace states
// themselves.  (Exp gate on the wide kernels: the dq pass reads the packed
// states, and this region stays unused.)
float* bw_states_f32(const mlstm_fw_desc_t* d2, void* workspace, float* region) {
  if (packed_layout(d2) || d2->precision == MLSTM_PREC_F64) return region;
  return ws_ptrs(d2, workspace).C;
}

}  // extern "C"

namespace {

// saved: the caller holds the forward's H and per-row m and normaliser, so
// only the chunk states are recomputed.
int bw_recompute(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
                 const float* f_pre, const float* C0, const float* n0, const float* m0, const void* dH,
                 void* workspace, size_t workspace_bytes, void* stream, bool saved) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->S > 0 && (!Q || !K || !V || !i_pre || !f_pre || !dH)) return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n0, m0, nullptr, nullptr)) != MLSTM_OK) return st;
  for (const void* x : {Q, K, V, dH})
    if (x && !aligned(x, 16)) return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, C0, n0, m0})) != MLSTM_OK) return st;
  const mlstm_fw_desc_t d2 = bw_fw_desc(desc);
  const BwLayout l = bw_layout(&d2);
  if (!workspace || workspace_bytes < l.total || !aligned(workspace, 256)) return MLSTM_E_WORKSPACE;
  if (desc->S == 0) return MLSTM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool ex = desc->gate == MLSTM_GATE_EXP;
  auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const WsPtrs fw = ws_ptrs(&d2, workspace);
  // Chunk states for the gradient stage.  On the wide kernels the packed
  // states feed the intra-chunk recompute (exp gate), and the dq pass reads
  // them packed too (both gates).  Float64: narrowed to float32.  The
  // generic kernels' float32 states are read in place (bw_states_f32).
  st = run_states(&d2, K, V, i_pre, f_pre, C0, n0, m0, fw, nullptr, nullptr, nullptr, s, nullptr, true);
  const bool convert = d2.precision == MLSTM_PREC_F64;
  if (st == MLSTM_OK)
    st = unpack_states(&d2, fw, convert ? at(l.Cst) : nullptr, ex ? at(l.nst) : nullptr, ex ? at(l.mst) : nullptr, s);
  if (st == MLSTM_OK && ex && !saved) {
    if (bw_delta_in_recompute(&d2))
      st = run_hintra(&d2, Q, K, V, i_pre, f_pre, fw, nullptr, at(l.mrows), at(l.den), s, dH,
                      desc->h_dtype == MLSTM_BF16, at(l.ginvz), at(l.gdelta));
    else
      st = run_hintra(&d2, Q, K, V, i_pre, f_pre, fw, at(l.H), at(l.mrows), at(l.den), s);
  }
  return st;
}

// H_saved, m_saved, den_saved: the forward's H and per-row m and normaliser
// (saved recompute), or null (the recompute's own).
int bw_grads(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
             const float* f_pre, const float* C0, const float* n0, const void* dH, float* dQ, float* dK, float* dV,
             float* d_i, float* d_f, float* dC0, float* dn0, float* dm0, void* workspace, size_t workspace_bytes,
             void* stream, const float* H_saved, const float* m_saved, const float* den_saved) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->S > 0 && (!Q || !K || !V || !i_pre || !f_pre || !dH || !dQ || !dK || !dV || !d_i || !d_f))
    return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n0, dn0, dm0, nullptr)) != MLSTM_OK) return st;
  for (const void* x : {Q, K, V, dH, static_cast<const void*>(dQ), static_cast<const void*>(dK),
                        static_cast<const void*>(dV)})
    if (x && !aligned(x, 16)) return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, C0, n0, d_i, d_f, dC0, dn0, dm0})) != MLSTM_OK) return st;
  const mlstm_fw_desc_t d2 = bw_fw_desc(desc);
  const BwLayout l = bw_layout(&d2);
  if (!workspace || workspace_bytes < l.total || !aligned(workspace, 256)) return MLSTM_E_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const bool ex = desc->gate == MLSTM_GATE_EXP;
  auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  mlstm::BwParams p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.i_pre = i_pre;
  p.f_pre = f_pre;
  p.dH = dH;
  const bool saved = ex && H_saved;
  p.delta_ready = !saved && bw_delta_in_recompute(&d2);
  p.G_packed = nullptr;  // set by the launcher where the row-tile recurrence runs
  p.H = saved ? H_saved : (ex && !p.delta_ready ? at(l.H) : nullptr);
  p.m_rows = saved ? m_saved : (ex ? at(l.mrows) : nullptr);
  p.den_rows = saved ? den_saved : (ex ? at(l.den) : nullptr);
  p.C_states = bw_states_f32(&d2, workspace, at(l.Cst));
  p.C_packed = packed_layout(&d2) ? reinterpret_cast<const uint16_t*>(ws_ptrs(&d2, workspace).C) : nullptr;
  p.n_states = ex ? at(l.nst) : nullptr;
  p.m_states = ex ? at(l.mst) : nullptr;
  p.C0 = C0;
  p.n0 = n0;
  p.gb = at(l.gb);
  p.gsrc = at(l.gsrc);
  p.ginvz = ex ? at(l.ginvz) : nullptr;
  p.gdelta = ex ? at(l.gdelta) : nullptr;
  p.dC_states = at(l.dC);
  p.dn_states = ex ? at(l.dn) : nullptr;
  p.qdq = at(l.qdq);
  p.kdk = at(l.kdk);
  p.gate_tot = at(l.gtot);
  p.dS_tiles = desc->qkv_dtype == MLSTM_BF16 ? at(l.dS) : nullptr;
  p.nseg = l.nseg;
  p.cps = l.cps;
  p.seg_C = l.nseg > 1 ? at(l.seg) : nullptr;
  p.seg_n = l.nseg > 1 && ex ? at(l.segn) : nullptr;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.d_i = d_i;
  p.d_f = d_f;
  // dm0 needs dC0 and dn0: the workspace holds them when the caller does not ask
  p.dC0 = dC0 ? dC0 : (dm0 ? at(l.dC0) : nullptr);
  p.dn0 = dn0 ? dn0 : (dm0 ? at(l.dn0) : nullptr);
  p.dm0 = dm0;
  p.scale = resolve_scale(desc);
  p.eps = desc->eps;
  p.BH = desc->B * desc->NH;
  p.S = desc->S;
  p.DK = desc->DHQK;
  p.DV = desc->DHV;
  p.L = d2.chunk_size;
  p.Nc = (d2.S + d2.chunk_size - 1) / d2.chunk_size;
  p.qkv_bf16 = desc->qkv_dtype == MLSTM_BF16;
  p.dh_bf16 = desc->h_dtype == MLSTM_BF16;
  const hipError_t e = mlstm::launch_bw(p, !ex, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLSTM_OK : MLSTM_E_HIP;
}

// The checks of mlstm_chunkwise_bw, before anything is launched.
int check_bw_args(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
                  const float* f_pre, const float* C0, const float* n0, const float* m0, const void* dH, float* dQ,
                  float* dK, float* dV, float* d_i, float* d_f, float* dC0, float* dn0, float* dm0,
                  void* workspace, size_t workspace_bytes) {
  int st = validate_desc(desc);
  if (st != MLSTM_OK) return st;
  if (desc->S > 0 && (!Q || !K || !V || !i_pre || !f_pre || !dH || !dQ || !dK || !dV || !d_i || !d_f))
    return MLSTM_E_NULLPTR;
  if ((st = check_sig_nulls(desc, n0, m0, dn0, dm0)) != MLSTM_OK) return st;
  for (const void* x : {Q, K, V, dH, static_cast<const void*>(dQ), static_cast<const void*>(dK),
                        static_cast<const void*>(dV)})
    if (x && !aligned(x, 16)) return MLSTM_E_ALIGN;
  if ((st = check_f32_ptrs({i_pre, f_pre, C0, n0, m0, d_i, d_f, dC0, dn0, dm0})) != MLSTM_OK) return st;
  const mlstm_fw_desc_t d2 = bw_fw_desc(desc);
  if (!workspace || workspace_bytes < bw_layout(&d2).total || !aligned(workspace, 256)) return MLSTM_E_WORKSPACE;
  return MLSTM_OK;
}

}  // namespace

extern "C" {

int mlstm_bw_recompute(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V,
                       const float* i_pre, const float* f_pre, const float* C0, const float* n0, const float* m0,
                       const void* dH, void* workspace, size_t workspace_bytes, void* stream) {
  return bw_recompute(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, dH, workspace, workspace_bytes, stream, false);
}

int mlstm_bw_grads(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V, const float* i_pre,
                   const float* f_pre, const float* C0, const float* n0, const void* dH, float* dQ, float* dK,
                   float* dV, float* d_i, float* d_f, float* dC0, float* dn0, float* dm0, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return bw_grads(desc, Q, K, V, i_pre, f_pre, C0, n0, dH, dQ, dK, dV, d_i, d_f, dC0, dn0, dm0, workspace,
                  workspace_bytes, stream, nullptr, nullptr, nullptr);
}

int mlstm_chunkwise_bw_saved(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V,
                             const float* i_pre, const float* f_pre, const float* C0, const float* n0,
                             const float* m0, const float* H, const float* m_rows, const float* den_rows,
                             const void* dH, float* dQ, float* dK, float* dV, float* d_i, float* d_f, float* dC0,
                             float* dn0, float* dm0, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_bw_args(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, dH, dQ, dK, dV, d_i, d_f, dC0, dn0, dm0,
                         workspace, workspace_bytes);
  if (st != MLSTM_OK) return st;
  const bool ex = desc->gate == MLSTM_GATE_EXP;
  if (ex) {
    if (desc->h_dtype != MLSTM_F32) return MLSTM_E_UNSUPPORTED;  // H is read as float32
    if (desc->S > 0 && (!H || !m_rows || !den_rows)) return MLSTM_E_NULLPTR;
    if (H && !aligned(H, 16)) return MLSTM_E_ALIGN;
    if ((st = check_f32_ptrs({m_rows, den_rows})) != MLSTM_OK) return st;
  } else if (H || m_rows || den_rows) {
    return MLSTM_E_UNSUPPORTED;  // the sig gate has no normaliser terms
  }
  st = bw_recompute(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, dH, workspace, workspace_bytes, stream, true);
  if (st != MLSTM_OK) return st;
  return bw_grads(desc, Q, K, V, i_pre, f_pre, C0, n0, dH, dQ, dK, dV, d_i, d_f, dC0, dn0, dm0, workspace,
                  workspace_bytes, stream, ex ? H : nullptr, m_rows, den_rows);
}

int mlstm_chunkwise_bw(const mlstm_fw_desc_t* desc, const void* Q, const void* K, const void* V,
                       const float* i_pre, const float* f_pre, const float* C0, const float* n0, const float* m0,
                       const void* dH, float* dQ, float* dK, float* dV, float* d_i, float* d_f, float* dC0,
                       float* dn0, float* dm0, void* workspace, size_t workspace_bytes, void* stream) {
  // all checks of both stages before anything is launched
  int st = check_bw_args(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, dH, dQ, dK, dV, d_i, d_f, dC0, dn0, dm0,
                         workspace, workspace_bytes);
  if (st != MLSTM_OK) return st;
  st = mlstm_bw_recompute(desc, Q, K, V, i_pre, f_pre, C0, n0, m0, dH, workspace, workspace_bytes, stream);
  if (st != MLSTM_OK) return st;
  return mlstm_bw_grads(desc, Q, K, V, i_pre, f_pre, C0, n0, dH, dQ, dK, dV, d_i, d_f, dC0, dn0, dm0, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"
