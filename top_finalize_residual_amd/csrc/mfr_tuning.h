/*
 * mfr_tuning.h - launch override of libmoe_finalize_rmsnorm, for tests,
 * sweeps and tuning. Not part of the public C ABI
 * (include/moe_finalize_rmsnorm.h): production callers never need it, and
 * every entry point picks its launch shape by itself.
 *
 * The override belongs to the calling thread: it applies to the later calls
 * of the entry points (and to moe_finalize_rmsnorm_path) made from that
 * thread only, so one thread's choice cannot change the launch shape, and
 * with it the last bit of normed_out, of a call made by another thread.
 * It takes precedence over the MFR_PATH environment variable.
 */
#ifndef MFR_TUNING_H
#define MFR_TUNING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Cache policy of the output stores. AUTO writes through (sc1) once both
 * outputs pass 12 MiB, and at decode sizes (up to 64 tokens) when the output
 * is bf16; otherwise it writes back. The two non-temporal
 * encodings (nt, and nt with sc1) exist for the fused op with exactly eight
 * slots and bf16 output, on the grid paths; any other launch takes the
 * automatic policy instead. */
enum mfr_store_policy {
    MFR_STORE_AUTO = 0,
    MFR_STORE_WRITE_BACK = 1,
    MFR_STORE_WRITE_THROUGH = 2,
    MFR_STORE_NONTEMPORAL = 3,
    MFR_STORE_NONTEMPORAL_WRITE_THROUGH = 4
};

/* Which token each workgroup of a grid path takes. The hardware hands the
 * workgroups of a dispatch to the eight XCDs in turn, so with the default
 * order neighbouring tokens run on different XCDs; XCD_RANGES gives each
 * XCD one contiguous range of tokens instead. Results are identical. */
enum mfr_token_order {
    MFR_ORDER_DEFAULT = 0,
    MFR_ORDER_XCD_RANGES = 1
};

/* path: 0 = automatic, else an mfr_path value (MFR_PATH_TOKEN,
 * MFR_PATH_STREAM or MFR_PATH_PERSIST; a path that cannot serve a shape
 * falls back to the automatic one for that call).
 * vectors_per_thread: 0 = automatic, else 1..4 (16-byte vectors of each row
 * handled per thread, so the workgroup size follows from H; a value whose
 * workgroup would exceed the kernel's limit, or that the chosen path does not
 * take, falls back to automatic).
 * store_policy: an mfr_store_policy value.
 * Returns MFR_ERR_ARG (nothing changes) for values outside those ranges,
 * else MFR_OK. residual_out is bit-identical under every override;
 * normed_out can differ in the last bit between workgroup shapes, whose
 * sum-of-squares reduction trees differ. */
int mfr_tuning_force_launch(int path, int vectors_per_thread, int store_policy);

/* Workgroups per CU, for the calling thread: 0 = automatic, else at most
 * that many. On the persistent path the grid is that times the CU count
 * (automatic: as many as fit at once), and never more than T. On the grid
 * paths the launch reserves enough dynamic LDS that no more than that many
 * workgroups fit on a CU; where the kernel's registers already allow no
 * more, or the cap cannot be expressed in LDS, the launch is unchanged, so a
 * large value means no cap. Automatic there: 2 for the stream path's
 * 3-vector kernels of the fused op with bf16 or FP8 output, at H above 5120
 * from T = 2048 on; else no cap. Returns
 * MFR_ERR_ARG for a negative value, else MFR_OK. */
int mfr_tuning_force_residency(int workgroups_per_cu);

/* Token order of the grid paths for the calling thread: an mfr_token_order
 * value. Returns MFR_ERR_ARG for other values, else MFR_OK. */
int mfr_tuning_force_token_order(int order);

#ifdef __cplusplus
}
#endif

#endif /* MFR_TUNING_H */
