/*
 * mlstm_tfla.h - C ABI of the MI355X (gfx950) chunkwise mLSTM forward pass,
 * its backward pass and the recurrent (decode) step.
 *
 * What is computed.  The forward pass of the mLSTM cell (matrix memory C
 * updated by an outer product, exponential input gate, normaliser n and
 * max-state stabiliser m; "xLSTM: the NX-AI repository behind the extended
 * LSTM architecture", section "Exponential gating, matrix memory, and why the
 * kernels decide everything"), evaluated in the chunkwise-parallel form with a
 * second level of tiling inside each chunk ("Tiled Flash Linear Attention:
 * More Efficient Linear RNN and xLSTM Kernels", abstract).  Per head, with
 * s = qk_scale, lf_t = log sigmoid(f_t):
 *
 *   exp gate:  m_t = max(lf_t + m_{t-1}, i_t)
 *              C_t = e^{lf_t + m_{t-1} - m_t} C_{t-1} + e^{i_t - m_t} k_t v_t^T
 *              n_t = e^{lf_t + m_{t-1} - m_t} n_{t-1} + e^{i_t - m_t} k_t
 *              h_t = s C_t^T q_t / (max(|s n_t . q_t|, e^{-m_t}) + eps)
 *   sig gate:  C_t = sigmoid(f_t) C_{t-1} + sigmoid(i_t) k_t v_t^T
 *              h_t = s C_t^T q_t                      (no n, no m)
 *
 * The two-stage split (an inter-chunk recurrence that materialises the state
 * entering every chunk, then an intra-chunk parallel stage that reads those
 * states) follows the parallel-stage interface listed on the
 * "flash-xlstm-exp 0.1.0" page (section "Usage": Q, K, V, input and forget
 * gates, per-chunk C/n/m states and chunk_size in; H plus per-row n and m
 * out).  mlstm_chunkwise_fw runs both stages.
 *
 * Conventions for every entry point.
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) on
 *     the current HIP device; sizes are element counts implied by the
 *     descriptor.  Tensors are contiguous, row-major:
 *        Q, K      (B, NH, S, DHQK)   qkv_dtype
 *        V         (B, NH, S, DHV)    qkv_dtype
 *        i_pre     (B, NH, S)         float32   input-gate pre-activation
 *        f_pre     (B, NH, S)         float32   forget-gate pre-activation
 *        C0, C_out (B, NH, DHQK, DHV) float32   (rows follow k, columns v)
 *        n0, n_out (B, NH, DHQK)      float32   exp gate only
 *        m0, m_out (B, NH)            float32   exp gate only
 *        H         (B, NH, S, DHV)    h_dtype
 *     Q, K, V and H must be 16-byte aligned; everything else 4-byte aligned.
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates no device memory and keeps no mutable global state, except
 *     for mlstm_chunkwise_fw_noalloc's static workspace (one array per GPU,
 *     part of the loaded code object).  Inputs are never written.  Outputs
 *     must not alias inputs.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Results are ready when the stream has finished.
 *   - Every call validates all arguments on the host before it launches
 *     anything and returns a status code; nothing is launched when the status
 *     is not MLSTM_OK.  A failed launch returns MLSTM_E_HIP.
 *   - Readings where the method leaves a step open: the scale s multiplies
 *     the query at readout (states are built from raw k, v); the forget gate
 *     applies at every step including the first; m starts at m0 (0 if m0 is
 *     NULL); eps is added after the max.
 */
#ifndef MLSTM_TFLA_H
#define MLSTM_TFLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLSTM_ABI_VERSION 11

typedef enum {
  MLSTM_OK = 0,
  MLSTM_E_NULLPTR = 1,     /* a required pointer is NULL                       */
  MLSTM_E_SHAPE = 2,       /* B, NH, S, DHQK or DHV out of the supported set   */
  MLSTM_E_CHUNK = 3,       /* chunk_size or tile sizes unsupported             */
  MLSTM_E_DTYPE = 4,       /* unknown dtype code                               */
  MLSTM_E_UNSUPPORTED = 5, /* a combination the library does not implement    */
  MLSTM_E_WORKSPACE = 6,   /* workspace missing or smaller than required       */
  MLSTM_E_HIP = 7,         /* a HIP launch or runtime call failed              */
  MLSTM_E_ALIGN = 8,       /* a pointer violates its alignment requirement     */
  MLSTM_E_ARG = 9          /* other invalid argument (gate, precision, eps...) */
} mlstm_status_t;

typedef enum { MLSTM_F32 = 0, MLSTM_BF16 = 1 } mlstm_dtype_t;
typedef enum { MLSTM_GATE_EXP = 0, MLSTM_GATE_SIG = 1 } mlstm_gate_t;

/* Arithmetic of the three contractions whose left operand is computed on the
 * fly (P = scores x decay in P.V, the carried state C in Q.C, and the gated
 * keys in K^T.V).  With bf16 inputs the raw Q, K, V enter the matrix cores
 * unchanged; the computed operand is rounded to nearest-even in one of two
 * ways, and every product accumulates in fp32:
 *   MLSTM_PREC_SPLIT: the operand is carried as a hi + lo pair of bf16
 *                     values (two MFMA passes, about 16 significant bits).
 *                     Default.
 *   MLSTM_PREC_F16:   a single bf16 rounding of the operand (one pass).
 *   MLSTM_PREC_F64:   everything (gates, scores, contractions, chunk states)
 *                     in fp64, on the fp64 matrix cores (the intra-chunk
 *                     stage at DHQK 512 on the vector units); for rows whose
 *                     sums cancel too strongly for fp32 accumulation.
 *                     Workspace states take 8 bytes per value.
 * SPLIT and F16 are the same for float32 inputs, which use fp32 matrix-core
 * instructions. */
typedef enum { MLSTM_PREC_SPLIT = 0, MLSTM_PREC_F16 = 1, MLSTM_PREC_F64 = 2 } mlstm_prec_t;

/* Which kernels mlstm_chunkwise_fw runs.
 *   MLSTM_SCHED_TWO_STAGE: the two stages (inter-chunk recurrence writing the
 *       state entering every chunk to the workspace, then the intra-chunk
 *       stage reading them back), as mlstm_fw_states + mlstm_fw_hintra.
 *   MLSTM_SCHED_FUSED: one launch: a chunk walker per head and 128-column
 *       slice of V carries its part of the state from chunk to chunk in
 *       registers and forms the gate terms of each chunk from i_pre and
 *       f_pre itself; no chunk state is written and no workspace is used
 *       (the TFLA page lists avoiding the states' round trip as a planned
 *       follow-up of its two-kernel design).  Needs bf16 inputs,
 *       MLSTM_PREC_SPLIT, DHQK = 256, DHV a multiple of 128 and
 *       chunk_size <= 512; otherwise MLSTM_E_UNSUPPORTED.  The stage-wise
 *       calls (mlstm_fw_states, mlstm_fw_hintra, mlstm_fw_unpack_states)
 *       reject this schedule.
 *   MLSTM_SCHED_AUTO: the library's choice: FUSED where it covers the shape
 *       and tile_lq and tile_lkv are 0 (it is the faster path on the
 *       7B-shaped workloads, for both gates), TWO_STAGE otherwise.  The
 *       workspace size still covers the two stages, and stage-wise calls run
 *       them. */
typedef enum {
  MLSTM_SCHED_AUTO = 0,
  MLSTM_SCHED_TWO_STAGE = 1,
  MLSTM_SCHED_FUSED = 2,
  MLSTM_SCHED_BLOCKED = 3
} mlstm_schedule_t;

/* How the two-stage schedule hands the chunk states from stage one to stage
 * two (the quantised-state follow-up on the "flash-xlstm-exp 0.1.0" page,
 * "Upgrade roadmap", item 3, applied to the hand-off):
 *   MLSTM_STATES_SPLIT: each value as a bf16 hi + lo pair, 4 bytes, the
 *       split the intra-chunk kernel feeds to the matrix cores.  Default.
 *   MLSTM_STATES_I16:   int16 codes, 2 bytes a value, with one
 *       power-of-two float32 scale per 16 x 32 block of the state (between
 *       its largest magnitude over 32767 and twice that; codes round half to
 *       even).
 *       The intra-chunk kernel turns each code into the exact hi + lo pair
 *       of code * scale, so the only added error is the coding step, at most
 *       half a scale per value: max |dH| 3e-3 on the 7B-shaped exp workload
 *       (CPU measurement), inside the 2e-2 bound.  Needs bf16 inputs,
 *       MLSTM_PREC_SPLIT, the wide family with DHQK 128 or 256 and DHV 256
 *       or 512, and a schedule other than MLSTM_SCHED_FUSED and
 *       MLSTM_SCHED_BLOCKED (else MLSTM_E_UNSUPPORTED).  Stage one then runs
 *       its row-tile kernel in one sequence segment.  It halves the chunk
 *       states of the workspace.  Under MLSTM_SCHED_AUTO the field applies
 *       where the two stages run (the fused walker hands no states over).
 *       The backward pass ignores it. */
typedef enum { MLSTM_STATES_SPLIT = 0, MLSTM_STATES_I16 = 1 } mlstm_state_codes_t;

typedef struct {
  int32_t B, NH;       /* batch, heads: >= 1                                   */
  int32_t S;           /* sequence length: >= 0, need not divide chunk_size;
                          S * max(DHQK, DHV) < 2^29 (else MLSTM_E_SHAPE)     */
  int32_t DHQK, DHV;   /* head dims: multiples of 64, at most 512 (float32
                          inputs: DHQK at most 256)                           */
  int32_t chunk_size;  /* L: power of two, 16..1024 (16 and 32: the generic
                          and float64 kernels, one tile per chunk)          */
  int32_t qkv_dtype;   /* mlstm_dtype_t of Q, K, V                             */
  int32_t h_dtype;     /* mlstm_dtype_t of H                                   */
  int32_t gate;        /* mlstm_gate_t                                         */
  int32_t precision;   /* mlstm_prec_t                                         */
  float qk_scale;      /* s; <= 0 selects 1/sqrt(DHQK)                         */
  float eps;           /* >= 0, added to the normaliser after the max          */
  int32_t tile_lq;     /* rows of the intra-chunk output tile; 0 = library    */
  int32_t tile_lkv;    /* key rows per intra-chunk step; 0 = library          */
  int32_t schedule;    /* mlstm_schedule_t; 0 = library choice                */
  int32_t block_chunks; /* MLSTM_SCHED_BLOCKED: chunks per block, >= 0; 0 =
                           library (a block's chunk states fill half of the
                           256 MB Infinity Cache); ignored otherwise        */
  int32_t state_codes; /* mlstm_state_codes_t; 0 = bf16 hi + lo pairs       */
  int32_t reserved;    /* must be zero                                        */
} mlstm_fw_desc_t;

/* ABI version of the loaded library (MLSTM_ABI_VERSION). */
int mlstm_abi_version(void);

/* Static text for a status code ("ok", "null pointer", ...). */
const char* mlstm_status_str(int status);

/* Host-only check of a descriptor (no pointers, no device calls).  Returns
 * MLSTM_OK or the first error found. */
int mlstm_fw_validate(const mlstm_fw_desc_t* desc);

/* Number of chunks N_c = ceil(S / chunk_size) for a valid descriptor, else
 * -1. */
int64_t mlstm_fw_num_chunks(const mlstm_fw_desc_t* desc);

/* Which family of kernels mlstm_chunkwise_fw runs for a valid descriptor
 * (host-only query):
 *   MLSTM_FAMILY_GENERIC  64-row tiles, float32 row-major chunk states, bf16
 *                         (bf16 inputs) or fp32 (float32 inputs) operands
 *   MLSTM_FAMILY_WIDE     bf16 inputs with DHQK in {128, 256} and DHV in
 *                         {256, 512}, tile_lq 0 or 64 (or 128 when the
 *                         chunk holds 128 rows): 512-thread intra-chunk
 *                         workgroups,
 *                         bf16 operands, chunk states in the packed operand
 *                         layout
 *   MLSTM_FAMILY_F64      MLSTM_PREC_F64: fp64 kernels on the fp64 matrix
 *                         cores (the intra-chunk stage at DHQK 512 on the
 *                         vector units)
 *   MLSTM_FAMILY_FUSED    the fused chunk walker (see mlstm_schedule_t):
 *                         bf16 operands, state carried in registers
 * This is the family mlstm_chunkwise_fw runs.  The stage-wise calls run
 * GENERIC, WIDE or F64 kernels: they reject a descriptor whose schedule is
 * MLSTM_SCHED_FUSED, and run the two stages for an MLSTM_SCHED_AUTO
 * descriptor that reports FUSED here.  Returns the negated status code for an
 * invalid descriptor. */
typedef enum {
  MLSTM_FAMILY_GENERIC = 0,
  MLSTM_FAMILY_WIDE = 1,
  MLSTM_FAMILY_F64 = 2,
  MLSTM_FAMILY_FUSED = 3,
  MLSTM_FAMILY_BLOCKED = 4
} mlstm_family_t;
int mlstm_fw_kernel_family(const mlstm_fw_desc_t* desc);

/* Bytes of device workspace that the forward pass needs for `desc`: the
 * stabilised state entering every chunk plus the final state, i.e. N_c + 1
 * states per head of DHQK x DHV values, DHQK normaliser values and one
 * max-state (exp gate), each region 256-byte aligned; 4 bytes per value, 8
 * with MLSTM_PREC_F64; with MLSTM_STATES_I16 the chunk states take 2 bytes
 * per value plus one more region of 4 bytes per 16 x 32 block of each state
 * (its scale).  For MLSTM_FAMILY_WIDE it also holds per-position gate
 * terms, written by stage one and read by stage two (12 bytes per position
 * and head for the exp gate, 8 for the sig gate), and 4 bytes per chunk
 * boundary and head for the stabilisers of sequence segments that stage one
 * may run side by side (two more 256-aligned regions).  A descriptor whose
 * schedule is MLSTM_SCHED_FUSED needs no workspace (0 bytes); under
 * MLSTM_SCHED_AUTO the size covers the two stages even where the fused
 * walker runs.  Returns 0 for an invalid descriptor.  The storage order inside
 * the workspace belongs to the library (the chunk states are kept in the
 * operand order of the kernels that read them); mlstm_fw_unpack_states
 * returns the states as plain float32. */
size_t mlstm_fw_workspace_bytes(const mlstm_fw_desc_t* desc);

/* Full forward pass: stage one (states) then stage two (H) on `workspace`,
 * or the fused chunk walker (see mlstm_schedule_t).
 *   C0, n0, m0   may be NULL: zero initial state (m0 = 0).  For the sig gate
 *                n0 and m0 must be NULL.
 *   C_out, n_out, m_out  may be NULL: that final state is not written.  For
 *                the sig gate n_out and m_out must be NULL.  The final state
 *                follows the stabiliser convention above: the true memory is
 *                C_out * e^{m_out}.
 *   workspace    device buffer of at least mlstm_fw_workspace_bytes(desc)
 *                bytes, 256-byte aligned; it may be NULL only when that size
 *                is 0.  On return it holds the chunk states (see
 *                mlstm_fw_unpack_states) when the two-stage kernels ran;
 *                the fused walker (MLSTM_FAMILY_FUSED) leaves it untouched:
 *                the chunk states were never formed.
 * With S == 0 the call only copies the initial state to the outputs. */
int mlstm_chunkwise_fw(const mlstm_fw_desc_t* desc,
                       const void* Q, const void* K, const void* V,
                       const float* i_pre, const float* f_pre,
                       const float* C0, const float* n0, const float* m0,
                       void* H,
                       float* C_out, float* n_out, float* m_out,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/* mlstm_chunkwise_fw that also writes the per-row quantities of the
 * normalisation ("xLSTM: the NX-AI repository behind the extended LSTM
 * architecture", section "Exponential gating, matrix memory, and why the
 * kernels decide everything": the max-state m and the normaliser; the
 * "flash-xlstm-exp 0.1.0" page, section "Usage", lists per-row n and m among
 * the parallel stage's outputs), for mlstm_chunkwise_bw_saved:
 *   m_rows   (B, NH, S) float32, may be NULL: the max-state m_t
 *   den_rows (B, NH, S) float32, may be NULL: the stabilised normaliser
 *            s n_t . q_t before the max with e^{-m_t}
 * Exp gate only (with the sig gate both must be NULL: MLSTM_E_UNSUPPORTED).
 * Every schedule writes them, the fused walker included; other arguments,
 * checks and errors as mlstm_chunkwise_fw. */
int mlstm_chunkwise_fw_rows(const mlstm_fw_desc_t* desc,
                            const void* Q, const void* K, const void* V,
                            const float* i_pre, const float* f_pre,
                            const float* C0, const float* n0, const float* m0,
                            void* H,
                            float* C_out, float* n_out, float* m_out,
                            float* m_rows, float* den_rows,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* Size of the static workspace of mlstm_chunkwise_fw_noalloc (64 MiB). */
#define MLSTM_NOALLOC_WORKSPACE_BYTES (64u << 20)

/* mlstm_chunkwise_fw for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same forward pass, same arguments without the workspace,
 * which comes from a static device array of MLSTM_NOALLOC_WORKSPACE_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 * The call allocates nothing.  When the workspace of the kernels that run
 * exceeds that size the call is refused with MLSTM_E_WORKSPACE before
 * anything is launched: where the fused walker runs (schedule FUSED, or AUTO
 * on a shape it covers) it uses none, so every size fits; the two-stage
 * kernels need mlstm_fw_workspace_bytes(desc), mostly chunk states, so they
 * fit for small problems only.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, two host
 * threads) race and give wrong results; calls ordered on one stream are
 * safe.  Nothing in the array needs to start at zero (every region a kernel
 * reads is written earlier in the same call).  The first call on a device
 * looks up the array's device address (MLSTM_E_HIP if that fails). */
int mlstm_chunkwise_fw_noalloc(const mlstm_fw_desc_t* desc,
                               const void* Q, const void* K, const void* V,
                               const float* i_pre, const float* f_pre,
                               const float* C0, const float* n0, const float* m0,
                               void* H,
                               float* C_out, float* n_out, float* m_out,
                               void* stream);

/* Stage one, the inter-chunk recurrence: writes into `workspace` the
 * stabilised state entering each chunk c = 0..N_c-1 (entry 0 is the initial
 * state) and the final state (entry N_c).  Arguments as for
 * mlstm_chunkwise_fw; Q is not needed. */
int mlstm_fw_states(const mlstm_fw_desc_t* desc,
                    const void* K, const void* V,
                    const float* i_pre, const float* f_pre,
                    const float* C0, const float* n0, const float* m0,
                    void* workspace, size_t workspace_bytes,
                    float* C_out, float* n_out, float* m_out,
                    void* stream);

/* Stage two, the intra-chunk parallel pass: H from Q, K, V, the gates and the
 * chunk states that mlstm_fw_states left in `workspace` (same descriptor).
 * Optional per-row outputs (NULL = not written; exp gate only):
 *   m_rows   (B, NH, S) float32: the max-state m_t
 *   den_rows (B, NH, S) float32: the stabilised normaliser s n_t . q_t before
 *            the max with e^{-m_t} */
int mlstm_fw_hintra(const mlstm_fw_desc_t* desc,
                    const void* Q, const void* K, const void* V,
                    const float* i_pre, const float* f_pre,
                    const void* workspace, size_t workspace_bytes,
                    void* H, float* m_rows, float* den_rows,
                    void* stream);

/* The chunk states held in `workspace`, as float32:
 *   C_states (B, NH, N_c + 1, DHQK, DHV)   (may be NULL)
 *   n_states (B, NH, N_c + 1, DHQK)        (exp gate; may be NULL)
 *   m_states (B, NH, N_c + 1)              (exp gate; may be NULL)
 * Entry c is the state entering chunk c; entry N_c the final state.  For the
 * sig gate n_states and m_states must be NULL. */
int mlstm_fw_unpack_states(const mlstm_fw_desc_t* desc,
                           const void* workspace, size_t workspace_bytes,
                           float* C_states, float* n_states, float* m_states,
                           void* stream);

/* One time step of the recurrence above for every head, the decode step
 * (the "xLSTM: the NX-AI repository behind the extended LSTM architecture"
 * page, section "Exponential gating, matrix memory, and why the kernels
 * decide everything", lists a step kernel beside the chunkwise and sequence
 * kernels).  `desc` describes a one-token forward pass: S must be 1 (else
 * MLSTM_E_SHAPE); B, NH, DHQK, DHV, qkv_dtype, h_dtype, gate, qk_scale and
 * eps are used, the other fields only validated.
 *   q, k      (B, NH, DHQK)       qkv_dtype, 16-byte aligned
 *   v         (B, NH, DHV)        qkv_dtype, 16-byte aligned
 *   i_pre, f_pre (B, NH)          float32
 *   C_in, n_in, m_in  the state entering the step, in the stabilised
 *             convention of C_out / n_out / m_out of mlstm_chunkwise_fw (so a
 *             forward pass's final state continues here); NULL = zero state.
 *             C_in (B, NH, DHQK, DHV) float32, 16-byte aligned.
 *   h         (B, NH, DHV)        h_dtype, 16-byte aligned, required
 *   C_out     (B, NH, DHQK, DHV) float32, 16-byte aligned, required; it may
 *             be the same buffer as C_in (updated in place).
 *   n_out, m_out  may be NULL (not written); they must not be the same
 *             buffers as n_in, m_in (MLSTM_E_ARG): every workgroup of a head
 *             reads n_in and m_in while one of them writes the new values.
 * For the sig gate n_in, m_in, n_out and m_out must be NULL.  The call is
 * bound by memory: it reads and writes the float32 state once. */
int mlstm_recurrent_step(const mlstm_fw_desc_t* desc,
                         const void* q, const void* k, const void* v,
                         const float* i_pre, const float* f_pre,
                         const float* C_in, const float* n_in, const float* m_in,
                         void* h,
                         float* C_out, float* n_out, float* m_out,
                         void* stream);

/* int8 block-quantised memory state for the decode step (the
 * "flash-xlstm-exp 0.1.0" page, section "Upgrade roadmap", lists a quantised
 * fp8/int8 state for long-context inference).  C is held as
 *   Cq (B, NH, DHQK, DHV) int8 codes and
 *   Cs (B, NH, DHV / 64, DHQK) float32 scales, one per block of 64
 *      consecutive values of a row: Cs[b][h][j][r] scales
 *      Cq[b][h][r][64 j .. 64 j + 63] (block-major, so that a run of rows
 *      moves in 16-byte pieces);
 * the block represents Cq * Cs.  A block x encodes as code =
 * round-half-even(x * 127 / amax), amax = max |x|, with scale amax / 127
 * (codes and scale 0 when amax = 0); the error is at most half a scale.  n
 * and m stay float32.
 *
 * mlstm_recurrent_step_q8: mlstm_recurrent_step on an encoded state.  The
 * step decodes the state, updates it in float32, reads h from the updated
 * values (before they are encoded again) and writes the encoded update.
 *   Cq_in, Cs_in   both NULL (zero state) or both given; Cq_in 4-byte and
 *                  Cs_in 16-byte aligned (likewise Cq_out, Cs_out).
 *   Cq_out, Cs_out required; they may be Cq_in, Cs_in (updated in place).
 *   Everything else as for mlstm_recurrent_step.
 * mlstm_state_q8_encode / _decode: a float32 state (B, NH, DHQK, DHV), such as
 *   C_out of mlstm_chunkwise_fw, to the encoded form and back (B, NH, DHQK
 *   and DHV from `desc`, which must be valid; S is not used). */
int mlstm_recurrent_step_q8(const mlstm_fw_desc_t* desc,
                            const void* q, const void* k, const void* v,
                            const float* i_pre, const float* f_pre,
                            const int8_t* Cq_in, const float* Cs_in,
                            const float* n_in, const float* m_in,
                            void* h,
                            int8_t* Cq_out, float* Cs_out,
                            float* n_out, float* m_out,
                            void* stream);
int mlstm_state_q8_encode(const mlstm_fw_desc_t* desc, const float* C, int8_t* Cq, float* Cs, void* stream);
int mlstm_state_q8_decode(const mlstm_fw_desc_t* desc, const int8_t* Cq, const float* Cs, float* C, void* stream);

/* Bytes of device workspace that mlstm_chunkwise_bw needs for `desc`: the
 * two-stage forward workspace, the recomputed forward quantities (chunk
 * states as float32, and for the exp gate H in float32 plus the per-row m and
 * normaliser), per-position gate terms, the state gradient after every
 * chunk (N_c states of DHQK x DHV float32 values per head, plus DHQK values
 * for the exp gate) and, for bf16 inputs, the weighted score gradients of
 * every pair of 64-row tiles in a chunk (64 x 64 float32 each), which one
 * gradient kernel hands to another.  Returns 0 for an invalid descriptor. */
size_t mlstm_bw_workspace_bytes(const mlstm_fw_desc_t* desc);

/* Backward pass: the gradients of sum(dH * H) with respect to the inputs of
 * mlstm_chunkwise_fw, for the same descriptor and inputs.  The pages print no
 * backward pass; this is the derivative of the forward pass above (the
 * "xLSTM: the NX-AI repository behind the extended LSTM architecture" page,
 * section "Exponential gating, matrix memory, and why the kernels decide
 * everything"), organised in chunks as the "Tiled Flash Linear Attention:
 * More Efficient Linear RNN and xLSTM Kernels" abstract describes for
 * training.  The max-state m is held constant: with eps = 0, H does not
 * depend on m and the gradient is exact; with eps > 0 it is the gradient at
 * fixed m.
 *   Q, K, V, i_pre, f_pre, C0, n0, m0   as for mlstm_chunkwise_fw.
 *   dH        (B, NH, S, DHV)  h_dtype, 16-byte aligned: the incoming gradient.
 *   dQ, dK    (B, NH, S, DHQK) float32, 16-byte aligned, required.
 *   dV        (B, NH, S, DHV)  float32, 16-byte aligned, required.
 *   d_i, d_f  (B, NH, S)       float32, required: gradients of i_pre, f_pre.
 *   dC0       (B, NH, DHQK, DHV) float32, may be NULL: gradient of C0 (of
 *             the zero state when C0 is NULL), in C0's stabilised convention.
 *   dn0       (B, NH, DHQK)    float32, may be NULL (exp gate only).
 *   dm0       (B, NH)          float32, may be NULL (exp gate only).
 *   workspace device buffer of at least mlstm_bw_workspace_bytes(desc) bytes,
 *             256-byte aligned; its contents on return belong to the library.
 * The forward quantities the gradient needs are recomputed with the two-stage
 * kernels whatever desc->schedule says (the fused walker forms neither chunk
 * states nor per-row normalisers); desc->precision applies to that
 * recomputation.  The gradient does not depend on how the sequence is cut
 * into chunks, so the backward picks its own: chunks of
 * min(max(chunk_size, 64), Lmax) rows, Lmax = 128 when B * NH * DHQK / 64 is
 * at least 256 (the chip's CU count) and 256 otherwise; the results agree
 * with those of any other cut to rounding.  (At 65536 tokens, 8 heads and
 * chunk 1024 the cut at 256 is 6 % faster than at 128 and 10 % faster than
 * at 512; at the 7B-shaped 64 heads the cut at 128 is 7 % faster than at
 * 512.)  The gradient kernels accumulate in float32: with bf16
 * inputs on bf16 matrix cores (Q, K, V raw, every computed operand as a bf16
 * hi + lo pair), with float32 inputs on fp32 matrix cores.  No gradient
 * flows in through the final state.  For the sig gate n0,
 * m0, dn0 and dm0 must be NULL.  Outputs must not alias inputs.  With S == 0
 * only dC0, dn0 and dm0 are written (zeros). */
int mlstm_chunkwise_bw(const mlstm_fw_desc_t* desc,
                       const void* Q, const void* K, const void* V,
                       const float* i_pre, const float* f_pre,
                       const float* C0, const float* n0, const float* m0,
                       const void* dH,
                       float* dQ, float* dK, float* dV,
                       float* d_i, float* d_f,
                       float* dC0, float* dn0, float* dm0,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/* mlstm_chunkwise_bw from the forward's own outputs: the gradient's row
 * terms (1/z and delta) come from H, m_rows and den_rows as
 * mlstm_chunkwise_fw_rows wrote them for the same descriptor and inputs,
 * so of the forward only the chunk states are recomputed (the intra-chunk
 * recompute is skipped).  Exp gate: desc->h_dtype must be MLSTM_F32
 * (MLSTM_E_UNSUPPORTED otherwise; H is read as float32, dH is float32 too);
 *   H        (B, NH, S, DHV) float32, 16-byte aligned, required
 *   m_rows   (B, NH, S) float32, required
 *   den_rows (B, NH, S) float32, required
 * Sig gate: the gradient has no normaliser terms, the three must be NULL
 * (MLSTM_E_UNSUPPORTED otherwise) and the call is mlstm_chunkwise_bw.  The
 * gradient agrees with mlstm_chunkwise_bw's to rounding (the row terms are
 * formed from the stored H instead of the recomputed one).  Other
 * arguments, workspace size, checks and errors as mlstm_chunkwise_bw. */
int mlstm_chunkwise_bw_saved(const mlstm_fw_desc_t* desc,
                             const void* Q, const void* K, const void* V,
                             const float* i_pre, const float* f_pre,
                             const float* C0, const float* n0, const float* m0,
                             const float* H, const float* m_rows, const float* den_rows,
                             const void* dH,
                             float* dQ, float* dK, float* dV,
                             float* d_i, float* d_f,
                             float* dC0, float* dn0, float* dm0,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* The two stages of mlstm_chunkwise_bw, for callers that time or schedule
 * them apart.  Same arguments as mlstm_chunkwise_bw; the same descriptor,
 * inputs and initial state must be given to both, and the workspace must not
 * change in between.
 *   mlstm_bw_recompute: the forward quantities the gradient needs, into the
 *       workspace (two-stage forward kernels: chunk states, and for the exp
 *       gate the per-row m and normaliser, with the row terms of the
 *       gradient that read dH: 1/z and delta = -(dh . h) / z * sign(den)
 *       where |den| > e^{-m}, else 0).  On the wide kernels (bf16 inputs,
 *       DHQK 128 or 256, DHV 256 or 512) the intra-chunk kernel forms those
 *       row terms in its epilogue and H is never stored; elsewhere H is
 *       stored in float32 and the gradient stage forms them.  dH is
 *       required (as in mlstm_chunkwise_bw).
 *   mlstm_bw_grads: the gradient kernels on that workspace (bf16 inputs:
 *       bf16 matrix cores, computed operands as bf16 hi + lo pairs; float32
 *       inputs: fp32 matrix cores): per-position gate terms, the state-gradient recurrence
 *       over the chunks in reverse order, dQ, dK, dV per 64-row tile, and the
 *       gate gradients by a reverse scan over the sequence.  The workspace's
 *       forward quantities are only read; its other regions are scratch. */
int mlstm_bw_recompute(const mlstm_fw_desc_t* desc,
                       const void* Q, const void* K, const void* V,
                       const float* i_pre, const float* f_pre,
                       const float* C0, const float* n0, const float* m0,
                       const void* dH,
                       void* workspace, size_t workspace_bytes,
                       void* stream);
int mlstm_bw_grads(const mlstm_fw_desc_t* desc,
                   const void* Q, const void* K, const void* V,
                   const float* i_pre, const float* f_pre,
                   const float* C0, const float* n0,
                   const void* dH,
                   float* dQ, float* dK, float* dV,
                   float* d_i, float* d_f,
                   float* dC0, float* dn0, float* dm0,
                   void* workspace, size_t workspace_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_TFLA_H */
