"""Host-side model of the GEMV kernel's weight addressing (launch plan, task
split, cursors, clamping), used to prove on the CPU that every load of every
lane of every wave stays inside the weight buffer for a given call shape.

It restates, in Python, the integer arithmetic of plan() in q4gemv.hip and of
the cursor / load() code of gemv_kernel in q4_kernels.h; keep the two in step
(test_addressing.py runs it over the parity-test shapes and edge cases)."""
Q4K_BYTES = 144
Q40_PAIR = 36
U32 = 0xFFFFFFFF


def pow2ceil(v):
    p = 1
    while p < v:
        p <<= 1
    return p


def plan(M, K, rows, RR, moe, npairs_max, cus=256, bpc=2, wpb=8):
    upr = K // 64
    lg = 64 if upr >= 64 else pow2ceil(upr)
    upl = (upr + lg - 1) // lg
    rgw = 64 // lg
    nrg = (rows + RR - 1) // RR
    if moe:
        nrg = (nrg + rgw - 1) // rgw * rgw
        ntasks = 0
        tasks = npairs_max * (nrg // rgw)
    else:
        ntasks = (nrg + rgw - 1) // rgw
        tasks = ntasks
    blocks = min(cus * bpc, (tasks + wpb - 1) // wpb)
    blocks = max(1, blocks)
    return dict(upr=upr, lg=lg, upl=upl, rgw=rgw, nrg=nrg, ntasks=ntasks, nwaves=blocks * wpb)


def unit_off(fmt, u):
    return (u >> 2) * Q4K_BYTES if fmt == "q4k" else u * Q40_PAIR


def loads(fmt, M, N, K, RR, nmat, moe_experts=None, E=1, **kw):
    """Yield (matrix, byte offset, nbytes) of every load; moe_experts is the
    list of unique valid experts the in-kernel dedupe would produce."""
    moe = moe_experts is not None
    pl = plan(M, K, N, RR, moe, kw.get("npairs_max", 1), **{k: v for k, v in kw.items()
                                                             if k in ("cus", "bpc")})
    rb = (K // 256) * 144 if fmt == "q4k" else (K // 32) * 18
    upr, lg, upl, rgw = pl["upr"], pl["lg"], pl["upl"], pl["rgw"]
    u_last = upr - 1
    if moe:
        tpe = pl["nrg"] // rgw
        nu = len(moe_experts)
        ntasks = nu * tpe
    else:
        tpe = 1
        ntasks = pl["ntasks"]
    for gw in range(pl["nwaves"]):
        t0, t1, ts = gw, ntasks, pl["nwaves"]
        # cursors visited: the first one always, then every task < t1
        curs = []
        ue = t0 // tpe if moe else 0
        rgt = t0 - ue * tpe if moe else t0
        t, ui = t0, 0
        curs.append((t, ui, ue, rgt))
        while True:
            ui += 1
            if ui == upl:
                ui = 0
                t += ts
                rgt += ts
                if moe and rgt >= tpe:
                    ue += rgt // tpe
                    rgt -= (rgt // tpe) * tpe
            if t >= t1:
                break
            curs.append((t, ui, ue, rgt))
        for (t, ui, ue, rgt) in curs:
            for lane in range(64):
                gi, li = lane // lg, lane % lg
                u = li + ui * lg
                in_row = u <= u_last
                uoff = unit_off(fmt, li) + ui * unit_off(fmt, lg) if in_row else unit_off(fmt, u_last)
                g = (li & 3) if in_row else (u_last & 3)
                qoff = uoff + 16 + 32 * g if fmt == "q4k" else uoff
                R0 = rgt * rgw * RR
                ubase = moe_experts[min(ue, nu - 1)] * N if (moe and nu > 0) else 0
                R0c = max(0, min(R0, N - 1))
                lrow_max = N - 1 - R0c
                for r in range(RR):
                    # the lane part is 32-bit unsigned arithmetic in the kernel
                    lr = min(gi * RR + r + (R0 - R0c), lrow_max) & U32
                    ro = (lr * rb) & U32
                    sbase = (ubase + R0c) * rb
                    for mt in range(nmat):
                        if fmt == "q4k":
                            yield mt, sbase + ((ro + uoff) & U32), 16
                            yield mt, sbase + ((ro + qoff) & U32), 16
                            yield mt, sbase + ((ro + qoff) & U32) + 16, 16
                        else:
                            yield mt, sbase + ((ro + uoff) & U32), 16
                            yield mt, sbase + ((ro + uoff) & U32) + 16, 16
                            yield mt, sbase + ((ro + uoff) & U32) + 32, 4


def check(fmt, M, N, K, RR, nmat, moe_experts=None, E=1, **kw):
    rows_total = (E if moe_experts is not None else 1) * N
    rb = (K // 256) * 144 if fmt == "q4k" else (K // 32) * 18
    limit = rows_total * rb
    n = 0
    for mt, off, nb in loads(fmt, M, N, K, RR, nmat, moe_experts, E, **kw):
        assert 0 <= off and off + nb <= limit, (fmt, M, N, K, mt, off, nb, limit)
        n += 1
    return n
