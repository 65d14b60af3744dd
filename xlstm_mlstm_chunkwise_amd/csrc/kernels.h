// Launch interface between the C ABI (api.hip) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {

// Per-position gate terms in log2 units, (BH, S) float32 each (the gates
// kernel writes them; the wide-tile kernels read them).
struct GatesParams {
  const float* i_pre;
  const float* f_pre;
  float* gb2;   // in-chunk inclusive cumulative sum of log sigmoid(f)
  float* gu2;   // input term minus gb2
  float* gpm2;  // running maximum of gu2 within the chunk (exp gate)
  int BH, S, L, Nc;
};

struct StatesParams {
  const void* K;
  const void* V;
  const float* i_pre;
  const float* f_pre;
  const float* C0;  // may be null (zero state)
  const float* n0;  // may be null
  const float* m0;  // may be null
  float* C_states;  // (BH, Nc + 1, DK, DV), required
  float* n_states;  // (BH, Nc + 1, DK), exp gate
  float* m_states;  // (BH, Nc + 1), exp gate
  float* C_out;     // may be null
  float* n_out;
  float* m_out;
  const float* gb2;  // gate terms (wide-tile kernels only)
  const float* gu2;
  const float* gpm2;
  float* m_local;    // (BH, Nc + 1) stabiliser of segment-local runs, log2 units (wide family)
  int BH, S, DK, DV, L, Nc;
  int nseg, cps;     // sequence segments per head and chunks per segment (row-tile kernel)
  // Wide family only: also deliver the chunk states as float32 row-major
  // (BH, Nc + 1, DK, DV); with plain_only the packed copy may be skipped
  // (no intra-chunk kernel reads it).
  float* C_plain = nullptr;
  int plain_only = 0;
  // Chunk range [c_lo, c_hi) of this launch (c_hi < 0: Nc) and the chunk-state
  // slots per head (0: Nc + 1): the state entering chunk c sits at slot
  // c - c_lo, the one after the last chunk at slot c_hi - c_lo.  A launch over
  // part of the chunks starts from C0, n0, m0 and ends in C_out, n_out,
  // m_out (row-tile states kernel, one segment).
  int c_lo = 0, c_hi = -1, slots = 0;
  int nt_states = 1;  // non-temporal stores of the packed chunk states
  // Packed states as int16 codes (row-tile kernel, one segment) when set:
  // C_states then holds one code per value in the packed fragment order,
  // DK * DV int16 per state, and C_scales one power-of-two float32 scale per
  // 16 x 32 fragment, (DK / 16) * (DV / 32) per state (value = code * scale).
  float* C_scales = nullptr;
};

struct HintraParams {
  const void* Q;
  const void* K;
  const void* V;
  const float* i_pre;
  const float* f_pre;
  const float* C_states;
  const float* n_states;
  const float* m_states;
  void* H;
  float* m_rows;    // may be null
  float* den_rows;  // may be null
  const float* gb2;  // gate terms (wide-tile kernel only)
  const float* gu2;
  const float* gpm2;
  float scale;
  float eps;
  int BH, S, DK, DV, L, Nc;
  int h_bf16;    // 1: H is bf16, 0: float32
  int tile_lq;   // rows per workgroup: 64 or 128
  int tile_lkv;  // keys per step: 64 or 128
  // Chunk range and state slots as in StatesParams (wide kernel only).
  int c_lo = 0, c_hi = -1, slots = 0;
  int pair_tiles = 0;  // wide kernel: schedule row tiles p and NQT-1-p together
  // int16-coded chunk states (wide kernel; layout as in StatesParams) when set
  const float* C_scales = nullptr;
  // Backward recompute (wide kernel, exp gate, 64-row tiles): with dH set,
  // H is not stored; per row the kernel writes ginvz = 1 / (max(|den|, e^-m)
  // + eps) and gdelta = -(dh . h) ginvz sign(den) where |den| > e^-m, else 0.
  const void* dH = nullptr;
  int dh_bf16 = 0;
  float* ginvz = nullptr;
  float* gdelta = nullptr;
};

// Fused chunk walker: one workgroup per (head, 128-column slice of V) runs
// the chunks of its head in order with its part of the state in registers.
struct WalkParams {
  const void* Q;
  const void* K;
  const void* V;
  const float* i_pre;  // (BH, S) gate pre-activations; the walker forms the gate terms
  const float* f_pre;
  const float* C0;  // may be null (zero state)
  const float* n0;  // may be null
  const float* m0;  // may be null
  void* H;
  float* C_out;  // may be null
  float* n_out;
  float* m_out;
  float* m_rows = nullptr;    // (BH, S) per-row max-state m, may be null (exp gate)
  float* den_rows = nullptr;  // (BH, S) per-row normaliser before the max with e^{-m}, may be null
  float scale;
  float eps;
  int BH, S, DK, DV, L, Nc;
  int h_bf16;
};

// One time step of the recurrence for every head (decode).
struct StepParams {
  const void* q;  // (BH, DK), bf16 or float32
  const void* k;
  const void* v;  // (BH, DV)
  const float* i_pre;  // (BH)
  const float* f_pre;
  const float* C_in;  // (BH, DK, DV) float32, may be null (zero state); may equal C_out
  const float* n_in;  // (BH, DK), may be null
  const float* m_in;  // (BH), may be null
  void* h;            // (BH, DV), bf16 or float32
  float* C_out;       // required
  float* n_out;       // may be null; must not alias n_in
  float* m_out;       // may be null; must not alias m_in
  // int8 block-quantised state (q8 = 1): codes (BH, DK, DV) and one float32
  // scale per 64 values of a row, block-major (BH, DV / 64, DK); C_in /
  // C_out unused
  const int8_t* Cq_in;  // may be null (zero state); may equal Cq_out
  const float* Cs_in;   // null exactly when Cq_in is; may equal Cs_out
  int8_t* Cq_out;
  float* Cs_out;
  float scale;
  float eps;
  int BH, DK, DV;
  int qkv_bf16, h_bf16;
  int q8;
};

// Backward pass: gradients of <dH, H> (bw_kernels.hip).  The forward
// quantities it reads (row max-state and normaliser, H, the chunk states as
// float32 row-major) come from a recomputation by the forward kernels.
struct BwParams {
  const void* Q;  // (BH, S, DK), bf16 or float32
  const void* K;
  const void* V;  // (BH, S, DV)
  const float* i_pre;  // (BH, S)
  const float* f_pre;
  const void* dH;        // (BH, S, DV), bf16 or float32
  const float* H;        // (BH, S, DV) float32 (exp gate), or null when delta_ready
  int delta_ready;       // exp gate: the recompute already wrote ginvz and gdelta
  uint16_t* G_packed;    // the state gradients in the packed bf16 hi + lo layout of the chunk
                         // states (row-tile recurrence), in dC_states' space, or null
  const float* m_rows;   // (BH, S) exp gate
  const float* den_rows; // (BH, S) exp gate
  const float* C_states; // (BH, Nc + 1, DK, DV) float32 row-major: state entering each chunk
  const uint16_t* C_packed;  // the same states in the packed bf16 hi + lo layout, or null; the
                             // bf16 dq pass then reads these instead of C_states
  const float* n_states; // (BH, Nc + 1, DK) exp gate
  const float* m_states; // (BH, Nc + 1) exp gate
  const float* C0;       // may be null (for dm0)
  const float* n0;       // may be null
  float* gb;             // (BH, S) scratch: in-chunk sum of log sigmoid(f)
  float* gsrc;           // (BH, S) scratch: i (exp) or log sigmoid(i) (sig)
  float* ginvz;          // (BH, S) scratch: 1 / z (exp)
  float* gdelta;         // (BH, S) scratch: normaliser gradient (exp)
  float* dC_states;      // (BH, Nc, DK, DV) scratch: state gradient after each chunk
  float* dn_states;      // (BH, Nc, DK) scratch (exp)
  float* qdq;            // (BH, S) scratch
  float* kdk;            // (BH, S) scratch
  float* gate_tot;       // (BH, ceil(S / 1024) + 32) scratch: sums of q.dq - k.dk over blocks of
                         // positions, then 32 partial sums of dC0 . C0
  float* dS_tiles;       // (BH, Nc, L/64 (L/64 + 1) / 2, 64, 64) scratch: weighted dS of every
                         // (query tile, key tile <= it) pair, written by the dk pass, read by dq
  float* dQ;             // (BH, S, DK) float32
  float* dK;
  float* dV;             // (BH, S, DV) float32
  float* d_i;            // (BH, S)
  float* d_f;
  float* dC0;            // (BH, DK, DV), may be null
  float* dn0;            // (BH, DK), may be null (exp)
  float* dm0;            // (BH), may be null (exp); needs dC0 and dn0
  float scale;
  float eps;
  int BH, S, DK, DV, L, Nc;
  int qkv_bf16, dh_bf16;
  // Sequence segments of the row-tile state-gradient recurrence
  // (bw_dstate_segments): segment s walks chunks [s cps, (s + 1) cps) from
  // zero and leaves its state gradient at the segment's first chunk in
  // seg_C ((BH, nseg, DK * DV) float32, packed fragment-lane order) and
  // seg_n ((BH, nseg, DK), exp gate); the join kernels make them true.
  int nseg = 1, cps = 0;
  float* seg_C = nullptr;
  float* seg_n = nullptr;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_gates(const GatesParams& p, bool sig, hipStream_t stream);
bool walk_supported(int DK, int DV, int L, bool bf16_inputs, bool split);
// Workgroups the walker launches for a shape (heads x column slices).
long long walk_workgroups(int BH, int DV);
hipError_t launch_walk(const WalkParams& p, bool sig, hipStream_t stream);
hipError_t launch_step(const StepParams& p, bool sig, hipStream_t stream);
// int8 block encoding of a float32 state (BH, DK, DV) and back; scales
// block-major (BH, DV / 64, DK).
hipError_t launch_q8_encode(const float* C, int8_t* Cq, float* Cs, long long BH, int DK, int DV,
                            hipStream_t stream);
hipError_t launch_q8_decode(const int8_t* Cq, const float* Cs, float* C, long long BH, int DK, int DV,
                            hipStream_t stream);
hipError_t launch_bw(const BwParams& p, bool sig, hipStream_t stream);
// Segments of the backward's row-tile state-gradient recurrence for a shape
// (1 when its heads alone fill the CUs, or when another kernel runs it);
// *cps receives the chunks per segment.
int bw_dstate_segments(int BH, int DK, int DV, int Nc, bool bf16_inputs, int* cps);
hipError_t launch_states(const StatesParams& p, bool bf16_inputs, bool sig, bool split, hipStream_t stream);
hipError_t launch_hintra(const HintraParams& p, bool bf16_inputs, bool sig, bool split, hipStream_t stream);

// Wide-tile intra-chunk kernel (bf16 inputs, large head dims): whether it
// covers a shape, and its launch.
bool hintra_wide_supported(int DK, int DV, int L, int tile_lq, bool bf16_inputs);
hipError_t launch_hintra_wide(const HintraParams& p, bool sig, bool split, hipStream_t stream);

// Wide-tile states kernel: writes the chunk states in the packed fragment
// layout read by the wide intra-chunk kernel (as int16 codes when
// p.C_scales is set: row-tile kernel only, one segment).
hipError_t launch_states_wide(const StatesParams& p, bool sig, bool split, hipStream_t stream);
// Row-tile states kernel over the chunk range of p, one segment (the blocked
// forward schedule); rows_tile_rows(DK, DV) > 0 where it covers the shape.
int rows_tile_rows(int DK, int DV);
hipError_t launch_states_rows_range(const StatesParams& p, bool sig, bool split, hipStream_t stream);
// Float64 precision mode: both stages in fp64, states kept in fp64.  The
// states stage runs on the fp64 matrix cores; the intra-chunk stage does for
// DK of 64, 128 or 256 (launch_hintra_f64m) and on the vector ALUs otherwise.
hipError_t launch_states_f64(const StatesParams& p, bool bf16_inputs, bool sig, hipStream_t stream);
hipError_t launch_hintra_f64(const HintraParams& p, bool bf16_inputs, bool sig, hipStream_t stream);
hipError_t launch_narrow_f64(const void* src, float* dst, long long n, hipStream_t stream);
bool hintra_f64m_supported(int DK);
hipError_t launch_hintra_f64m(const HintraParams& p, bool bf16_inputs, bool sig, hipStream_t stream);
// Packed states (n_states x DK x DV) -> float32; scales non-null: the
// states are int16 codes with one scale per fragment (StatesParams::C_scales).
hipError_t launch_unpack_states(const void* packed, float* C, long long n_states, int DK, int DV,
                                hipStream_t stream, const float* scales = nullptr);

}  // namespace mlstm
