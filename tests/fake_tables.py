"""Task tables with made-up addresses for host-only plan checks (no memory
behind them: wt_plan_check and wt_plan_schedule never dereference shards)."""
from bf16_fp8_weight_amd import workloads as W


def fake_table(wt, wl, base=0x7F0000000000, gap=0, align=256, host=None):
    """Shard addresses laid out in table order from `base`, each shard start
    aligned to `align` plus `gap` extra bytes between shards."""
    addr = base
    tasks = []
    mem = wt.WT_MEM_PINNED_HOST if (host if host is not None else wl.shard_mem == "host") else wt.WT_MEM_DEVICE
    for oi, o in enumerate(wl.outputs):
        fused = len(o.parts) > 1
        for p in o.parts:
            shards = []
            for r in p.shard_rows:
                if r == 0:
                    shards.append((0, 0))
                    continue
                addr = -(-addr // align) * align
                shards.append((addr, r))
                addr += 2 * r * o.cols + gap
            tasks.append({
                "shards": shards, "shard_mem": mem, "cols": o.cols,
                "dtype": wt.WT_FP8_E4M3FN_B128 if o.kind == W.FP8 else wt.WT_BF16_COPY,
                "fusion_group": oi if fused else -1,
                "dst_offset": o.dst_offset, "scale_offset": o.scale_offset,
            })
    return wt.TaskTable(tasks)
